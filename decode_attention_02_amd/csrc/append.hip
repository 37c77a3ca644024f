// Append path: write each sequence's s_q new tokens into the paged latent cache, with the
// RoPE key rotated to the token's position, and expand just those tokens into every
// group's K/V (the steps right before decode: the latent comes from the down-projection
// and, on the GQA path, is expanded into G key/value heads — "GQLA: Attention latente
// ...", English abstract; gqla_attn.py docstring, GQA path).
//
// One workgroup takes 16 new tokens and one group: it stages the tokens' latent rows
// (c as stored, k_rope rotated in fp64 and rounded once to the data type) in LDS; the
// group-0 workgroups write the latent rows, and every workgroup computes its group's
// d_n + d_v projected features of the 16 tokens, one feature row per thread (the weight
// row is read once for all 16 tokens, the latent values are LDS broadcasts), and copies
// the rotated RoPE key into K. Small work (B * s_q tokens per step): plain fp32 VALU.
#include "device_common.h"
#include "gqla_internal.h"

#include <cmath>

namespace gqla {

namespace {

constexpr int kAppendTile = 16;   // new tokens per workgroup

// Eight consecutive values as fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8f(const bf16_t* p, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = bf16_to_f32(static_cast<bf16_t>(w[q] & 0xffffu));
    o[2 * q + 1] = bf16_to_f32(static_cast<bf16_t>(w[q] >> 16));
  }
}
__device__ __forceinline__ void load8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void append_tokens_kernel(AppendParams a, const T* c_new, const T* kr_new,
                                                            const T* w_uk, const T* w_uv, T* latent, T* expanded) {
  extern __shared__ __attribute__((aligned(16))) float s_row[];   // [kAppendTile][d_c + d_R]
  const int dq = a.dc + a.dr;
  const int dqk = a.dn + a.dr;
  const int g = blockIdx.y;
  const int n0 = blockIdx.x * kAppendTile;
  __shared__ int64_t s_dst[kAppendTile];   // latent row index (block * 64 + slot), -1 = skip
  if (threadIdx.x < kAppendTile) {
    const int n = n0 + threadIdx.x;
    int64_t dst = -1;
    if (n < a.n_tok) {
      const int b = n / a.s_q, i = n % a.s_q;
      const int L = a.ctx_lens[b];
      if (L >= a.s_q && L <= a.max_blocks * kBlock) {
        const int t = L - a.s_q + i;
        const int32_t id = a.block_table[static_cast<int64_t>(b) * a.max_blocks + t / kBlock];
        if (id >= 0 && id < a.num_blocks) dst = static_cast<int64_t>(id) * kBlock + t % kBlock;
      }
    }
    s_dst[threadIdx.x] = dst;
  }
  // Stage the rows: c as stored; RoPE pairs (k, k + d_R/2) rotated by t * theta^(-2k/d_R).
  const int half = a.dr / 2;
  for (int idx = threadIdx.x; idx < kAppendTile * dq; idx += blockDim.x) {
    const int j = idx / dq, e = idx % dq;
    const int n = n0 + j;
    float v = 0.f;
    if (n < a.n_tok) {
      if (e < a.dc) {
        v = Elt<T>::load(c_new, static_cast<int64_t>(n) * a.dc + e);
      } else {
        const int k = e - a.dc, kk = k % half;
        const int b = n / a.s_q, i = n % a.s_q;
        const double t = static_cast<double>(a.ctx_lens[b] - a.s_q + i);
        const double ang = t * pow(static_cast<double>(a.rope_theta), -2.0 * kk / a.dr);
        const double cs = cos(ang), sn = sin(ang);
        const double x1 = Elt<T>::load(kr_new, static_cast<int64_t>(n) * a.dr + kk);
        const double x2 = Elt<T>::load(kr_new, static_cast<int64_t>(n) * a.dr + kk + half);
        const double r = k < half ? x1 * cs - x2 * sn : x1 * sn + x2 * cs;
        T rounded;
        Elt<T>::store(&rounded, 0, static_cast<float>(r));
        v = Elt<T>::load(&rounded, 0);   // the value the cache will hold
      }
    }
    s_row[j * dq + e] = v;
  }
  __syncthreads();
  if (g == 0) {
    for (int idx = threadIdx.x; idx < kAppendTile * dq; idx += blockDim.x) {
      const int j = idx / dq, e = idx % dq;
      if (s_dst[j] >= 0) Elt<T>::store(latent, s_dst[j] * dq + e, s_row[j * dq + e]);
    }
  }
  if (expanded == nullptr) return;
  const int rows = a.dn + a.dv;
  for (int r = threadIdx.x; r < rows + a.dr; r += blockDim.x) {
    float acc[kAppendTile];
#pragma unroll
    for (int j = 0; j < kAppendTile; ++j) acc[j] = 0.f;
    if (r < rows) {
      const T* wrow = r < a.dn ? w_uk + (static_cast<int64_t>(g) * a.dn + r) * a.dc
                               : w_uv + (static_cast<int64_t>(g) * a.dv + (r - a.dn)) * a.dc;
      for (int c = 0; c < a.dc; c += 8) {   // d_c is a multiple of 8 (checked by the caller)
        float wv[8];
        load8f(wrow + c, wv);
#pragma unroll
        for (int j = 0; j < kAppendTile; ++j) {
          const float4 x0 = *reinterpret_cast<const float4*>(s_row + j * dq + c);
          const float4 x1 = *reinterpret_cast<const float4*>(s_row + j * dq + c + 4);
          acc[j] += wv[0] * x0.x + wv[1] * x0.y + wv[2] * x0.z + wv[3] * x0.w +
                    wv[4] * x1.x + wv[5] * x1.y + wv[6] * x1.z + wv[7] * x1.w;
        }
      }
    } else {   // RoPE key feature d_n + k: the rotated value itself
#pragma unroll
      for (int j = 0; j < kAppendTile; ++j) acc[j] = s_row[j * dq + a.dc + (r - rows)];
    }
    // Key feature f (nope rows, then RoPE) or value feature of slot s, in the expanded
    // chunk's slab layout (see gqla_expand_cache).
    const bool is_v = r >= a.dn && r < rows;
    const int f = r < a.dn ? r : (is_v ? r - a.dn : a.dn + (r - rows));
#pragma unroll
    for (int j = 0; j < kAppendTile; ++j) {
      const int64_t dst = s_dst[j];
      if (dst < 0) continue;
      const int64_t id = dst / kBlock;
      const int s = static_cast<int>(dst % kBlock);
      T* chunk = expanded + (id * a.G + g) * static_cast<int64_t>(kBlock) * (dqk + a.dv);
      int64_t off;
      if (is_v) {
        off = static_cast<int64_t>(kBlock) * dqk + (s / kHalf) * a.dv * kHalf + f * kHalf + s % kHalf;
      } else {
        const int sl = f / kSlab, w = min(kSlab, dqk - sl * kSlab);
        off = static_cast<int64_t>(sl) * kBlock * kSlab + s * w + f % kSlab;
      }
      Elt<T>::store(chunk, off, acc[j]);
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& a, const void* c_new, const void* kr_new, const void* w_uk,
                         const void* w_uv, void* latent, void* expanded, bool bf16, hipStream_t s) {
  const int tiles = (a.n_tok + kAppendTile - 1) / kAppendTile;
  dim3 grid(tiles, expanded != nullptr ? a.G : 1);
  const size_t lds = sizeof(float) * kAppendTile * (a.dc + a.dr);
  if (bf16) {
    auto k = append_tokens_kernel<bf16_t>;
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    k<<<grid, 256, lds, s>>>(a, static_cast<const bf16_t*>(c_new), static_cast<const bf16_t*>(kr_new),
                             static_cast<const bf16_t*>(w_uk), static_cast<const bf16_t*>(w_uv),
                             static_cast<bf16_t*>(latent), static_cast<bf16_t*>(expanded));
  } else {
    auto k = append_tokens_kernel<float>;
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    k<<<grid, 256, lds, s>>>(a, static_cast<const float*>(c_new), static_cast<const float*>(kr_new),
                             static_cast<const float*>(w_uk), static_cast<const float*>(w_uv),
                             static_cast<float*>(latent), static_cast<float*>(expanded));
  }
  return hipGetLastError();
}

}  // namespace gqla
