// Placeholder: tuned kernels not yet built; every shape takes the generic kernels.
#include "tuned.h"
namespace gqla {
bool tuned_absorb_supported(const gqla_dims*) { return false; }
int tuned_absorb_target_wgs(const gqla_dims*) { return 256; }
int tuned_absorb_min_blocks_per_split() { return 2; }
hipError_t launch_tuned_absorb(const AttnParams&, const gqla_dims*, hipStream_t) { return hipErrorNotSupported; }
bool tuned_absorb_query_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_absorb_query(const ProjParams&, const void*, const void*, const void*, void*, hipStream_t) { return hipErrorNotSupported; }
bool tuned_out_proj_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_out_proj(const ProjParams&, const float*, const void*, void*, hipStream_t) { return hipErrorNotSupported; }
bool tuned_expand_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_expand(const ProjParams&, const void*, const void*, const void*, const int32_t*, int64_t, int64_t, void*, hipStream_t) { return hipErrorNotSupported; }
}
