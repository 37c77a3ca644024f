// MFMA kernels for the production GQLA shapes (bf16 data, d_c = 512, d_R = 64).
#pragma once

#include "../../include/gqla.h"
#include "gqla_internal.h"

namespace gqla {

// GQA split-KV decode: bf16, d_qk in {128, 192}, d_v = 128, gs * s_q <= 32 (one or two
// 16-row MFMA tiles per group); the shared-RoPE layout needs d_R = 64.
bool tuned_gqa_supported(const gqla_dims* d);
int tuned_gqa_target_wgs();
int tuned_gqa_min_blocks_per_split();
hipError_t launch_tuned_gqa(const AttnParams& p, const gqla_dims* d, hipStream_t s);

// Absorb split-KV decode: bf16, d_c = 512, d_R = 64, H * s_q in {16, 32, 64, 128, 256, 512}.
bool tuned_absorb_supported(const gqla_dims* d);
int tuned_absorb_target_wgs(const gqla_dims* d);
int tuned_absorb_min_blocks_per_split();
int tuned_absorb_max_blocks_per_split();
hipError_t launch_tuned_absorb(const AttnParams& p, const gqla_dims* d, hipStream_t s);

bool tuned_absorb_query_supported(const gqla_dims* d);
hipError_t launch_tuned_absorb_query(const ProjParams& p, const void* q_nope, const void* q_rope,
                                     const void* w_uk, void* q_abs, hipStream_t s);
bool tuned_out_proj_supported(const gqla_dims* d);
hipError_t launch_tuned_out_proj(const ProjParams& p, const float* o_lat, const void* w_uv, void* out,
                                 hipStream_t s);
// Split combine fused with the value projection (absorb path): d_c = 512, d_v = 128, bf16,
// 2..64 splits.
bool tuned_combine_out_supported(const gqla_dims* d, int n_split);
hipError_t launch_tuned_combine_out(const ProjParams& p, const float* ws_o, const float* ws_lse, int n_split,
                                    float* o_lat, float* lse, const void* w_uv, void* out, hipStream_t s);
bool tuned_expand_supported(const gqla_dims* d);
hipError_t launch_tuned_expand(const ProjParams& p, const void* latent, const void* w_uk, const void* w_uv,
                               const int32_t* block_ids, int64_t n_blocks, int64_t num_blocks,
                               void* expanded, hipStream_t s);

}  // namespace gqla
