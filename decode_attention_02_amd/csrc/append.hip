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
  const int g = blockIdx.y;
  const int n0 = blockIdx.x * kAppendTile;
  const ExpandedLayout lay = expanded_layout(a.dn, a.dr, a.dv, a.G, a.rope_shared != 0);
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
        const double ang = t * a.inv_freq[kk];
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
  if (g == 0 && latent != nullptr) {
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
    // cache's slab layout (see gqla_expand_cache); a shared RoPE key goes to the block's
    // key area, written by group 0 only.
    const bool is_v = r >= a.dn && r < rows;
    const int f = r < a.dn ? r : (is_v ? r - a.dn : a.dn + (r - rows));
    const bool shared_key = !is_v && f >= lay.k_feats;
    if (shared_key && g != 0) continue;
#pragma unroll
    for (int j = 0; j < kAppendTile; ++j) {
      const int64_t dst = s_dst[j];
      if (dst < 0) continue;
      const int64_t id = dst / kBlock;
      const int s = static_cast<int>(dst % kBlock);
      T* blk = expanded + id * lay.block;
      T* chunk = blk + lay.rope + g * lay.chunk;
      if (is_v) {
        Elt<T>::store(chunk, static_cast<int64_t>(kBlock) * lay.k_feats + (s / kHalf) * a.dv * kHalf + f * kHalf + s % kHalf, acc[j]);
      } else if (!shared_key) {
        const int sl = f / kSlab, w = min(kSlab, lay.k_feats - sl * kSlab);
        Elt<T>::store(chunk, static_cast<int64_t>(sl) * kBlock * kSlab + s * w + f % kSlab, acc[j]);
      } else {
        const int fr = f - a.dn, sl = fr / kSlab, w = min(kSlab, a.dr - sl * kSlab);
        Elt<T>::store(blk, static_cast<int64_t>(sl) * kBlock * kSlab + s * w + fr % kSlab, acc[j]);
      }
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 with d_c % 32 == 0 and (d_n + d_v) % 16 == 0: the projections on MFMA. Workgroup
// (token tile, group, z < nz) has 4 waves, wave w taking the 16 stacked weight rows
// 16 * (4z + w) .. +16 of [W_UK^g ; W_UV^g]: K^T/V^T = W C^T with A = 16 weight rows x 32
// latent values and B = 32 latent values x 16 tokens, both read straight from global
// memory with every load of the wave in flight at once. The workgroups z = nz rotate the
// tile's keys, write the latent rows (group 0) and copy the keys into K, so that neither
// kind waits for the other's memory round trips (the step is latency-bound). With no
// expanded cache (the absorb path keeps only the latent) the grid is just those workgroups.
template <int DC>
__global__ __launch_bounds__(256) void append_tokens_mfma(AppendParams a, const bf16_t* c_new, const bf16_t* kr_new,
                                                          const bf16_t* w_uk, const bf16_t* w_uv, bf16_t* latent,
                                                          bf16_t* expanded, int nz) {
  constexpr int KS = DC / 32;
  const int dq = DC + a.dr;
  const ExpandedLayout lay = expanded_layout(a.dn, a.dr, a.dv, a.G, a.rope_shared != 0);
  const int g = blockIdx.y;
  const int n0 = blockIdx.x * kAppendTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  __shared__ int64_t s_dst[kAppendTile];
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
  const int rows = a.dn + a.dv;
  const int row0 = 16 * (4 * blockIdx.z + wave);
  // Issue every operand load of this wave first.
  const bool live_rows = static_cast<int>(blockIdx.z) < nz && row0 < rows;
  bf16x8 wa[KS], cb[KS];
  if (live_rows) {
    const int r = row0 + col;
    const bf16_t* wrow = r < a.dn ? w_uk + (static_cast<int64_t>(g) * a.dn + r) * DC
                                  : w_uv + (static_cast<int64_t>(g) * a.dv + (r - a.dn)) * DC;
    const int n = min(n0 + col, a.n_tok - 1);   // past the last token: re-read it, store nothing
    const bf16_t* crow = c_new + static_cast<int64_t>(n) * DC;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      wa[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks + 8 * grp);
      cb[ks] = *reinterpret_cast<const bf16x8*>(crow + 32 * ks + 8 * grp);
    }
  }
  __syncthreads();   // s_dst
  if (static_cast<int>(blockIdx.z) == nz) {
    if (a.rope_shared && g != 0) return;   // the shared key and the latent rows are group 0's
    // Group 0 copies the latent rows (when a latent cache is kept): their loads go out first
    // and their stores follow the rotation, so the two memory round trips overlap.
    constexpr int kCopies = kAppendTile * (DC / 8) / 256;
    static_assert(kAppendTile * (DC / 8) % 256 == 0, "whole 16-byte copies per thread");
    const bool write_latent = g == 0 && latent != nullptr;
    uint4 cp[kCopies];
    if (write_latent) {
#pragma unroll
      for (int u = 0; u < kCopies; ++u) {
        const int idx = threadIdx.x + 256 * u, j = idx / (DC / 8), c8 = idx % (DC / 8);
        const int n = min(n0 + j, a.n_tok - 1);   // past the last token: re-read it, store nothing
        cp[u] = *reinterpret_cast<const uint4*>(c_new + static_cast<int64_t>(n) * DC + 8 * c8);
      }
    }
    // The rotated keys of the tile (fp64 angle, rounded once), one rotation pair
    // (kk, kk + d_R/2) per thread and step, both of its sines from one sincos.
    __shared__ bf16_t s_rope[kAppendTile * 128];
    const int half = a.dr / 2;
    for (int idx = threadIdx.x; idx < kAppendTile * half; idx += blockDim.x) {
      const int j = idx / half, kk = idx % half;
      const int n = min(n0 + j, a.n_tok - 1);
      const int b = n / a.s_q, i = n % a.s_q;
      const double ang = static_cast<double>(a.ctx_lens[b] - a.s_q + i) * a.inv_freq[kk];
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double x1 = bf16_to_f32(kr_new[static_cast<int64_t>(n) * a.dr + kk]);
      const double x2 = bf16_to_f32(kr_new[static_cast<int64_t>(n) * a.dr + kk + half]);
      s_rope[j * a.dr + kk] = f32_to_bf16(static_cast<float>(x1 * cs - x2 * sn));
      s_rope[j * a.dr + kk + half] = f32_to_bf16(static_cast<float>(x1 * sn + x2 * cs));
    }
    if (write_latent) {
#pragma unroll
      for (int u = 0; u < kCopies; ++u) {
        const int idx = threadIdx.x + 256 * u, j = idx / (DC / 8), c8 = idx % (DC / 8);
        const int64_t dst = s_dst[j];
        if (dst >= 0) *reinterpret_cast<uint4*>(latent + dst * dq + 8 * c8) = cp[u];
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kAppendTile * a.dr; idx += blockDim.x) {
      const int j = idx / a.dr, k = idx % a.dr;
      const int64_t dst = s_dst[j];
      if (dst < 0) continue;
      if (expanded != nullptr) {
        const int64_t id = dst / kBlock;
        const int s = static_cast<int>(dst % kBlock);
        bf16_t* blk = expanded + id * lay.block;
        if (!a.rope_shared) {   // into this group's K
          const int f = a.dn + k, sl = f / kSlab, w = min(kSlab, lay.k_feats - sl * kSlab);
          blk[lay.rope + g * lay.chunk + static_cast<int64_t>(sl) * kBlock * kSlab + s * w + f % kSlab] = s_rope[idx];
        } else if (g == 0) {    // once, into the block's shared key area
          const int sl = k / kSlab, w = min(kSlab, a.dr - sl * kSlab);
          blk[static_cast<int64_t>(sl) * kBlock * kSlab + s * w + k % kSlab] = s_rope[idx];
        }
      }
      if (write_latent) latent[dst * dq + DC + k] = s_rope[idx];
    }
  }
  if (!live_rows) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks], cb[ks], acc, 0, 0, 0);
  // Lane holds rows row0 + 4*grp + r (r = 0..3) of token col.
  const int64_t dst = s_dst[col];
  if (dst < 0) return;
  const int64_t id = dst / kBlock;
  const int s = static_cast<int>(dst % kBlock);
  bf16_t* chunk = expanded + id * lay.block + lay.rope + g * lay.chunk;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * grp + r;
    int64_t off;
    if (row < a.dn) {
      const int sl = row / kSlab, w = min(kSlab, lay.k_feats - sl * kSlab);
      off = static_cast<int64_t>(sl) * kBlock * kSlab + s * w + row % kSlab;
    } else {
      const int f = row - a.dn;
      off = static_cast<int64_t>(kBlock) * lay.k_feats + (s / kHalf) * a.dv * kHalf + f * kHalf + s % kHalf;
    }
    chunk[off] = f32_to_bf16(acc[r]);
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& a, const void* c_new, const void* kr_new, const void* w_uk,
                         const void* w_uv, void* latent, void* expanded, bool bf16, hipStream_t s) {
  const int tiles = (a.n_tok + kAppendTile - 1) / kAppendTile;
  if (bf16 && a.dc == 512 && a.dr <= 128 && (a.dn + a.dv) % 16 == 0) {
    // Without an expanded cache only the rotation / latent-copy workgroups run (nz = 0).
    const int nz = expanded != nullptr ? (a.dn + a.dv + 63) / 64 : 0;
    dim3 grid(tiles, expanded != nullptr ? a.G : 1, nz + 1);
    append_tokens_mfma<512><<<grid, 256, 0, s>>>(a, static_cast<const bf16_t*>(c_new), static_cast<const bf16_t*>(kr_new),
                                                 static_cast<const bf16_t*>(w_uk), static_cast<const bf16_t*>(w_uv),
                                                 static_cast<bf16_t*>(latent), static_cast<bf16_t*>(expanded), nz);
    return hipGetLastError();
  }
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
