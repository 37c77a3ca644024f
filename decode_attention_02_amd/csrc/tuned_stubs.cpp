// Placeholder: tuned kernels not yet built; every shape takes the generic kernels.
#include "tuned.h"
namespace gqla {
bool tuned_absorb_query_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_absorb_query(const ProjParams&, const void*, const void*, const void*, void*, hipStream_t) { return hipErrorNotSupported; }
bool tuned_out_proj_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_out_proj(const ProjParams&, const float*, const void*, void*, hipStream_t) { return hipErrorNotSupported; }
bool tuned_expand_supported(const gqla_dims*) { return false; }
hipError_t launch_tuned_expand(const ProjParams&, const void*, const void*, const void*, const int32_t*, int64_t, int64_t, void*, hipStream_t) { return hipErrorNotSupported; }
}
