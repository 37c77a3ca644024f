// Small per-group projections of the MQA-absorb path on gfx950 MFMA (bf16 weights).
//
//   absorb query:  q_abs[b][i][h] = [ W_UK^g^T q_nope[b][i][h] ; q_rope[b][i][h] ]
//   value output:  out[b][i][h]   =   W_UV^g o_lat[b][i][h]
// (W_UK^g folded into the query, W_UV^g applied to the latent output: "GQLA: Attention
// latente ...", English abstract; gqla_attn.py docstring, MQA-absorb path.)
//
// Both are grouped GEMMs with few rows per group, bound by moving the queries, the
// latent outputs and the weights. A workgroup takes one group and 64 of its query rows
// (4 waves x 16), copies the group's weight matrix once into LDS (global_load_lds, in
// flight together with the row operands) and forms the transposed
// product so that each lane ends with 4 consecutive output features of one row
// (8-byte stores):
//   * absorb query: q_abs^T = W_UK^g^T q^T contracts over W_UK's row index, so the
//     weight operand is read transposed with ds_read_b64_tr_b16;
//   * value output: out^T = W_UV^g o_lat^T contracts over W_UV's contiguous column index
//     (ds_read_b128). The fp32 latent output is split into bf16 high and low parts
//     (two MFMAs) so the product keeps close to fp32 accuracy.
#include "device_common.h"
#include "gqla_internal.h"
#include "tuned.h"

namespace gqla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kDV = 128;
constexpr int kPadRow = kDC * 2 + 32;   // LDS row stride in bytes: rows shift by 8 banks
constexpr int kRowsPerWG = 64;

// Row rg of group g (0 <= rg < B * s_q * gs) is query row (b, i) = rg / gs of head
// g * gs + rg % gs; returns its index in [B][s_q][H].
__device__ __forceinline__ int64_t group_row(int rg, int g, int gs, int H) {
  return static_cast<int64_t>(rg / gs) * H + g * gs + rg % gs;
}

typedef __attribute__((address_space(3))) void lds_void;

// Copy a [rows][512] bf16 weight matrix into LDS rows of stride kPadRow: one
// global_load_lds_dwordx4 per 1 KiB row (lane l brings bytes 16l..16l+15), so the copy
// needs no registers and every wave's share is in flight at once. Waits for it.
__device__ __forceinline__ void stage_rows(char* lds, const bf16_t* src, int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  for (int r = wave; r < rows; r += waves)
    __builtin_amdgcn_global_load_lds(src + r * kDC + 8 * lane, (lds_void*)(lds + r * kPadRow), 16, 0, 0);
}

template <int DN>
__global__ __launch_bounds__(256) void absorb_query_kernel(ProjParams d, const bf16_t* q_nope, const bf16_t* q_rope,
                                                           const bf16_t* w_uk, bf16_t* q_abs) {
  __shared__ __attribute__((aligned(16))) char w[DN * kPadRow];
  const int g = blockIdx.y;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rg = blockIdx.x * kRowsPerWG + wave * 16 + col;   // this lane's row (B operand column)
  const bool live = rg < rows_g;
  const int64_t row = live ? group_row(rg, g, gs, d.H) : 0;
  constexpr int KS = DN / 32;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = live ? *reinterpret_cast<const bf16x8*>(q_nope + row * DN + 32 * ks + 8 * grp) : bf16x8{};
  stage_rows(w, w_uk + static_cast<int64_t>(g) * DN * kDC, DN);
  __builtin_amdgcn_s_waitcnt(0);   // queries and this wave's weight rows have landed
  __syncthreads();
  const int dq = kDC + kDR;
  // A operand (W^T, 16 latent features x 32 nope values): source lane `col` of each
  // 16-lane group supplies nope row 32*ks + 8*grp + 4*half + (col >> 2), features
  // 16*ct + 4*(col & 3); the transposed read hands lane (feature f, grp) 4 nope values.
  const int src_n = 8 * grp + (col >> 2);
  const int src_f = 4 * (col & 3);
#pragma unroll 4
  for (int ct = 0; ct < kDC / 16; ++ct) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const char* base = w + (32 * ks + src_n) * kPadRow + (16 * ct + src_f) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * kPadRow));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], acc, 0, 0, 0);
    }
    if (live) {
      bf16_t packed[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[k]);
      *reinterpret_cast<uint2*>(q_abs + row * dq + 16 * ct + 4 * grp) = *reinterpret_cast<uint2*>(packed);
    }
  }
  // RoPE part is a copy: 64 values = 8 chunks of 16 bytes per row.
  for (int i = threadIdx.x; i < kRowsPerWG * (kDR / 8); i += blockDim.x) {
    const int r = blockIdx.x * kRowsPerWG + i / (kDR / 8), c = i % (kDR / 8);
    if (r >= rows_g) continue;
    const int64_t rr = group_row(r, g, gs, d.H);
    *reinterpret_cast<uint4*>(q_abs + rr * dq + kDC + 8 * c) = *reinterpret_cast<const uint4*>(q_rope + rr * kDR + 8 * c);
  }
}

__global__ __launch_bounds__(256) void out_proj_kernel(ProjParams d, const float* o_lat, const bf16_t* w_uv, bf16_t* out) {
  __shared__ __attribute__((aligned(16))) char w[kDV * kPadRow];
  const int g = blockIdx.y;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rg = blockIdx.x * kRowsPerWG + wave * 16 + col;
  const bool live = rg < rows_g;
  const int64_t row = live ? group_row(rg, g, gs, d.H) : 0;
  // The lane's whole slice of its latent-output row (16 k-steps x 8 values), loaded up
  // front together with the weight copy so both are in flight at once.
  const float* o = o_lat + row * kDC + 8 * grp;
  f32x4 xo[kDC / 32][2];
#pragma unroll
  for (int ks = 0; ks < kDC / 32; ++ks) {
    xo[ks][0] = live ? *reinterpret_cast<const f32x4*>(o + 32 * ks) : f32x4{0.f, 0.f, 0.f, 0.f};
    xo[ks][1] = live ? *reinterpret_cast<const f32x4*>(o + 32 * ks + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  stage_rows(w, w_uv + static_cast<int64_t>(g) * kDV * kDC, kDV);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x4 acc[kDV / 16];
#pragma unroll
  for (int vt = 0; vt < kDV / 16; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int ks = 0; ks < kDC / 32; ++ks) {
    // B operand: 8 latent values of this lane's row, as bf16 high + low parts.
    bf16x8 hi, lo;
    const f32x4 x0 = xo[ks][0];
    const f32x4 x1 = xo[ks][1];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float x = k < 4 ? x0[k] : x1[k - 4];
      const __bf16 h = static_cast<__bf16>(x);
      hi[k] = h;
      lo[k] = static_cast<__bf16>(x - static_cast<float>(h));
    }
#pragma unroll
    for (int vt = 0; vt < kDV / 16; ++vt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(w + (16 * vt + col) * kPadRow + (32 * ks + 8 * grp) * 2);
      acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc[vt], 0, 0, 0);
      acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc[vt], 0, 0, 0);
    }
  }
  if (!live) return;
#pragma unroll
  for (int vt = 0; vt < kDV / 16; ++vt) {
    bf16_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[vt][k]);
    *reinterpret_cast<uint2*>(out + row * kDV + 16 * vt + 4 * grp) = *reinterpret_cast<uint2*>(packed);
  }
}

}  // namespace

bool tuned_absorb_query_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->rope_dim == kDR &&
         (d->nope_dim == 64 || d->nope_dim == 128);
}

hipError_t launch_tuned_absorb_query(const ProjParams& p, const void* q_nope, const void* q_rope, const void* w_uk,
                                     void* q_abs, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  dim3 grid((rows_g + kRowsPerWG - 1) / kRowsPerWG, p.G);
  const bf16_t* qn = static_cast<const bf16_t*>(q_nope);
  const bf16_t* qr = static_cast<const bf16_t*>(q_rope);
  const bf16_t* wk = static_cast<const bf16_t*>(w_uk);
  bf16_t* qa = static_cast<bf16_t*>(q_abs);
  if (p.dn == 128) absorb_query_kernel<128><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa);
  else absorb_query_kernel<64><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa);
  return hipGetLastError();
}

bool tuned_out_proj_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->v_dim == kDV;
}

hipError_t launch_tuned_out_proj(const ProjParams& p, const float* o_lat, const void* w_uv, void* out, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  dim3 grid((rows_g + kRowsPerWG - 1) / kRowsPerWG, p.G);
  out_proj_kernel<<<grid, 256, 0, s>>>(p, o_lat, static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(out));
  return hipGetLastError();
}

}  // namespace gqla
