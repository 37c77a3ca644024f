// Small per-group projections of the MQA-absorb path on gfx950 MFMA (bf16 weights).
//
//   absorb query:  q_abs[b][i][h] = [ W_UK^g^T q_nope[b][i][h] ; q_rope[b][i][h] ]
//   value output:  out[b][i][h]   =   W_UV^g o_lat[b][i][h]
// (W_UK^g folded into the query, W_UV^g applied to the latent output: "GQLA: Attention
// latente ...", English abstract; gqla_attn.py docstring, MQA-absorb path.)
//
// Both are grouped GEMMs with few rows per group and a 64-128 KiB weight per group, so
// at decode batch sizes they are latency-bound: the work is cut along the weight's
// output dimension as well as along the rows, so that even a single sequence spreads
// over dozens of workgroups, each holding only a slice of the weight. Both form the
// transposed product, so each lane ends with 4 consecutive output features of one row
// (8-byte stores):
//   * absorb query: q_abs^T = W_UK^g^T q^T contracts over W_UK's row index, so a
//     workgroup copies a [d_n][128] column slice of W_UK^g into LDS (global_load_lds)
//     and reads the weight operand transposed with ds_read_b64_tr_b16;
//   * value output: out^T = W_UV^g o_lat^T contracts over W_UV's contiguous column
//     index, so each single-wave workgroup keeps its 32 rows of W_UV^g in registers
//     (direct 16-byte loads) across the row tiles it visits. The fp32 latent output is
//     split into bf16 high and low parts (two MFMAs) so the product keeps close to fp32
//     accuracy.
// Workgroups are small (one wave; four for the absorbed query at large row counts) so the
// weight and row reads of a small batch spread over most CUs instead of a few.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kDV = 128;
constexpr int kSliceF = 128;     // latent features per absorb-query workgroup
constexpr int kMaxWGs = 2048;    // grid cap: larger row counts loop over row tiles

// Row rg of group g (0 <= rg < B * s_q * gs) is query row (b, i) = rg / gs of head
// g * gs + rg % gs; returns its index in [B][s_q][H].
__device__ __forceinline__ int64_t group_row(int rg, int g, int gs, int H) {
  return static_cast<int64_t>(rg / gs) * H + g * gs + rg % gs;
}

// LDS layout of the absorb-query weight slice: DN rows of 256 bytes (128 features),
// the 16-byte chunk c of row r stored at chunk c ^ swz(r). The transposed operand read
// touches 4 rows x 32 bytes per 16 lanes (rows 8 apart for the next 16 lanes); the XOR
// gives those rows distinct chunk pairs, so a 32-lane read covers all 64 banks once.
__device__ __forceinline__ int swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

// NW waves per workgroup, 16 rows each: 4 when the rows are many (the staged weight slice
// serves 64 rows), 1 when 64-row workgroups would leave most CUs idle.
template <int DN, int NW>
__global__ __launch_bounds__(NW * 64) void absorb_query_kernel(ProjParams d, const bf16_t* q_nope, const bf16_t* q_rope,
                                                               const bf16_t* w_uk, bf16_t* q_abs) {
  __shared__ __attribute__((aligned(16))) char w[DN * kSliceF * 2];
  constexpr int RW = 16 * NW;   // rows per workgroup pass
  const int g = blockIdx.z;
  const int f0 = blockIdx.x * kSliceF;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + RW - 1) / RW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  constexpr int KS = DN / 32;
  // Stage the [DN][128] slice: each global_load_lds_dwordx4 fills 1 KiB = 4 rows, lane l
  // landing at row 4i + l/16, stored chunk l%16, which holds source chunk (l%16)^swz(row).
  {
    const bf16_t* src = w_uk + static_cast<int64_t>(g) * DN * kDC + f0;
#pragma unroll
    for (int i = wave; i < DN / 4; i += NW) {
      const int r = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ swz(r);
      __builtin_amdgcn_global_load_lds(src + r * kDC + 8 * c, (lds_void*)(w + 1024 * i), 16, 0, 0);
    }
  }
  const int dq = kDC + kDR;
  // A operand (W^T, 16 latent features x 32 nope values): source lane `col` of each
  // 16-lane group supplies nope row 32*ks + 8*grp + 4*half + (col >> 2), features
  // 16*ct + 4*(col & 3); the transposed read hands lane (feature f, grp) 4 nope values.
  const int src_n = 8 * grp + (col >> 2);
  const int src_b = 8 * (col & 3);   // byte offset inside the 32-byte feature tile
  bool staged = false;
  for (int rt = blockIdx.y; rt < n_rt; rt += gridDim.y) {
    const int rg = rt * RW + wave * 16 + col;   // this lane's row (B operand column)
    const bool live = rg < rows_g;
    const int64_t row = group_row(live ? rg : rows_g - 1, g, gs, d.H);   // past the end: re-read the last row
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(q_nope + row * DN + 32 * ks + 8 * grp);
    if (!staged) {
      __builtin_amdgcn_s_waitcnt(0);   // queries and this wave's weight rows have landed
      __syncthreads();
      staged = true;
    }
#pragma unroll
    for (int ct = 0; ct < kSliceF / 16; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r0 = 32 * ks + src_n, r1 = r0 + 4;
        const int b = 32 * ct + src_b;
        const char* p0 = w + r0 * 256 + ((((b >> 4) ^ swz(r0)) << 4) | (b & 15));
        const char* p1 = w + r1 * 256 + ((((b >> 4) ^ swz(r1)) << 4) | (b & 15));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
        const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], acc, 0, 0, 0);
      }
      if (live) {
        bf16_t packed[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[k]);
        *reinterpret_cast<uint2*>(q_abs + row * dq + f0 + 16 * ct + 4 * grp) = *reinterpret_cast<uint2*>(packed);
      }
    }
    // The RoPE part is a copy (64 values = 8 chunks of 16 bytes per row), done by the
    // first feature slice.
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < RW * (kDR / 8); i += blockDim.x) {
        const int r = rt * RW + i / (kDR / 8), c = i % (kDR / 8);
        if (r >= rows_g) continue;
        const int64_t rr = group_row(r, g, gs, d.H);
        *reinterpret_cast<uint4*>(q_abs + rr * dq + kDC + 8 * c) =
            *reinterpret_cast<const uint4*>(q_rope + rr * kDR + 8 * c);
      }
    }
  }
}

__global__ __launch_bounds__(64) void out_proj_kernel(ProjParams d, const float* o_lat, const bf16_t* w_uv, bf16_t* out) {
  const int g = blockIdx.y;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + 15) / 16;
  const int lane = threadIdx.x, wave = blockIdx.z;   // one wave per workgroup: its 32 rows of W_UV^g
  const int col = lane & 15, grp = lane >> 4;
  // A operand, kept for every row tile: W_UV^g rows 32*wave + 16*t + col, latent values
  // 32*ks + 8*grp .. +8.
  bf16x8 wa[2][kDC / 32];
  {
    const bf16_t* wsrc = w_uv + (static_cast<int64_t>(g) * kDV + 32 * wave + col) * kDC + 8 * grp;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < kDC / 32; ++ks)
        wa[t][ks] = *reinterpret_cast<const bf16x8*>(wsrc + 16 * t * kDC + 32 * ks);
  }
  for (int rt = blockIdx.x; rt < n_rt; rt += gridDim.x) {
    const int rg = rt * 16 + col;
    const bool live = rg < rows_g;
    // Lanes past the last row read the last row (loads stay unconditional, so the whole
    // row slice is in flight at once) and store nothing.
    const int64_t row = group_row(live ? rg : rows_g - 1, g, gs, d.H);
    const float* o = o_lat + row * kDC + 8 * grp;
    f32x4 xo[kDC / 32][2];
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks) {
      xo[ks][0] = *reinterpret_cast<const f32x4*>(o + 32 * ks);
      xo[ks][1] = *reinterpret_cast<const f32x4*>(o + 32 * ks + 4);
    }
    // Keep the scheduler from spreading these loads over the MFMA chain (it would, to save
    // registers, and every wait in between would be a full memory round trip).
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks) {
      // B operand: 8 latent values of this lane's row, as bf16 high + low parts.
      bf16x8 hi, lo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float x = xo[ks][k >> 2][k & 3];
        const __bf16 h = static_cast<__bf16>(x);
        hi[k] = h;
        lo[k] = static_cast<__bf16>(x - static_cast<float>(h));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[t][ks], hi, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[t][ks], lo, acc[t], 0, 0, 0);
      }
    }
    if (live) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16_t packed[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[t][k]);
        *reinterpret_cast<uint2*>(out + row * kDV + 32 * wave + 16 * t + 4 * grp) = *reinterpret_cast<uint2*>(packed);
      }
    }
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
  const int per_row = (kDC / kSliceF) * p.G;
  const bool wide = static_cast<int64_t>((rows_g + 63) / 64) * per_row >= kNumCUs;
  const int n_rt = wide ? (rows_g + 63) / 64 : (rows_g + 15) / 16;
  dim3 grid(kDC / kSliceF, std::max(1, std::min(n_rt, kMaxWGs / per_row)), p.G);
  const bf16_t* qn = static_cast<const bf16_t*>(q_nope);
  const bf16_t* qr = static_cast<const bf16_t*>(q_rope);
  const bf16_t* wk = static_cast<const bf16_t*>(w_uk);
  bf16_t* qa = static_cast<bf16_t*>(q_abs);
  if (wide) {
    if (p.dn == 128) absorb_query_kernel<128, 4><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa);
    else absorb_query_kernel<64, 4><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa);
  } else {
    if (p.dn == 128) absorb_query_kernel<128, 1><<<grid, 64, 0, s>>>(p, qn, qr, wk, qa);
    else absorb_query_kernel<64, 1><<<grid, 64, 0, s>>>(p, qn, qr, wk, qa);
  }
  return hipGetLastError();
}

bool tuned_out_proj_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->v_dim == kDV;
}

hipError_t launch_tuned_out_proj(const ProjParams& p, const float* o_lat, const void* w_uv, void* out, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  const int n_rt = (rows_g + 15) / 16;
  // One wave per workgroup (32 rows of W_UV^g, z = which 32), so that the weight and
  // latent-output reads spread over many CUs. Each wave loads its 32 KiB of W_UV^g once;
  // with many row tiles a wave visits at least 4 of them so that weight reloads stay small
  // next to the latent-output reads.
  const int want = std::max((n_rt + 3) / 4, 256 / p.G);
  dim3 grid(std::max(1, std::min({n_rt, want, kMaxWGs / p.G})), p.G, kDV / 32);
  out_proj_kernel<<<grid, 64, 0, s>>>(p, o_lat, static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(out));
  return hipGetLastError();
}

}  // namespace gqla
