// Generic (any-shape) kernels of the GQLA decode path, fp32 or bf16 data, fp32 math.
//
// These cover every dims combination that fits the LDS budget, in particular the fp32
// layer shapes; the MFMA kernels in the other files take the DeepSeek-V3 / LLaMA-3
// production shapes. Work per thread is plain VALU arithmetic read straight from
// global memory: simple, exact in fp32, not tuned.
#include "device_common.h"
#include "gqla_internal.h"

#include <cmath>

namespace gqla {

constexpr int kGenRows = 16;      // query rows per workgroup
constexpr int kGenThreads = 256;

size_t generic_attn_lds_bytes(int dk, int dvo) {
  return sizeof(float) * (static_cast<size_t>(kGenRows) * (dk + kBlock + dvo) + 3 * kGenRows);
}

// Key feature f of slot t: plain strides for the latent, or the expanded cache's slabs
// (features [32s, 32s + w_s) of all 64 slots stored slot-major, w_s the slab's width),
// features [0, k_own) in the group chunk at `base`, the rest (a shared RoPE key) in the
// block's key area at `rbase`.
template <typename T>
__device__ __forceinline__ float kv_k_load(const AttnParams& p, const T* base, const T* rbase, int t, int f) {
  if (p.k_slab == 0) return Elt<T>::load(base, static_cast<int64_t>(t) * p.k_ts + static_cast<int64_t>(f) * p.k_fs);
  const bool own = f < p.k_own;
  const int ff = own ? f : f - p.k_own;
  const int nf = own ? p.k_own : p.dk - p.k_own;
  const int s = ff / p.k_slab;
  const int w = min(p.k_slab, nf - s * p.k_slab);
  return Elt<T>::load(own ? base : rbase, static_cast<int64_t>(s) * kBlock * p.k_slab + t * w + (ff - s * p.k_slab));
}

__device__ __forceinline__ int64_t kv_v_index(const AttnParams& p, int t, int f) {
  return p.v_off + static_cast<int64_t>(t / kHalf) * p.v_half + static_cast<int64_t>(t % kHalf) * p.v_ts +
         static_cast<int64_t>(f) * p.v_fs;
}

// One workgroup = (split, row tile, sequence x kv head). Online softmax over the
// 64-token blocks of its split: scores to LDS, row statistics, rescaled accumulation.
template <typename T>
__global__ __launch_bounds__(kGenThreads) void generic_attn_split(AttnParams p) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int r0 = blockIdx.y * kGenRows;
  const int b = blockIdx.z / p.kv_heads;
  const int kvh = blockIdx.z % p.kv_heads;
  const int rows_total = p.heads_per_kv * p.s_q;
  const int nr = min(kGenRows, rows_total - r0);
  const T* q = static_cast<const T*>(p.q);
  const T* kv = static_cast<const T*>(p.kv);

  float* sq = smem;                        // [kGenRows][dk]
  float* ss = sq + kGenRows * p.dk;        // [kGenRows][64]
  float* so = ss + kGenRows * kBlock;      // [kGenRows][dvo]
  float* sm = so + kGenRows * p.dvo;       // running max
  float* sl = sm + kGenRows;               // running sum
  float* sa = sl + kGenRows;               // rescale factor of the current block

  const int L = p.ctx_lens[b];
  // Metadata the launch cannot honour makes the rows NaN instead of reading past
  // the table or silently dropping tokens.
  bool bad = (L < p.s_q) || (L > p.max_blocks * kBlock) ||
             ((L + kBlock - 1) / kBlock > p.n_split * p.blocks_per_split);

  for (int idx = tid; idx < nr * p.dk; idx += kGenThreads) {
    const int r = idx / p.dk, f = idx % p.dk, rr = r0 + r;
    const int i = rr / p.heads_per_kv, h = kvh * p.heads_per_kv + rr % p.heads_per_kv;
    sq[idx] = Elt<T>::load(q, (static_cast<int64_t>(b * p.s_q + i) * p.H + h) * p.dk + f);
  }
  for (int idx = tid; idx < nr * p.dvo; idx += kGenThreads) so[idx] = 0.f;
  if (tid < kGenRows) { sm[tid] = -INFINITY; sl[tid] = 0.f; }
  __syncthreads();

  const int nblk = bad ? 0 : (L + kBlock - 1) / kBlock;
  const int blk_lo = split * p.blocks_per_split;
  const int blk_hi = min(nblk, blk_lo + p.blocks_per_split);
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const int32_t id = p.block_table[static_cast<int64_t>(b) * p.max_blocks + blk];
    if (id < 0 || id >= p.num_blocks) { bad = true; break; }   // uniform across the group
    const T* rbase = kv + static_cast<int64_t>(id) * p.block_stride;
    const T* base = rbase + p.kv_off + kvh * p.kvh_stride;
    for (int idx = tid; idx < nr * kBlock; idx += kGenThreads) {
      const int r = idx / kBlock, t = idx % kBlock, rr = r0 + r;
      const int n = L - p.s_q + 1 + rr / p.heads_per_kv;
      float s = -INFINITY;
      if (blk * kBlock + t < n) {
        float acc = 0.f;
        for (int f = 0; f < p.dk; ++f)
          acc += sq[r * p.dk + f] * kv_k_load(p, base, rbase, t, f);
        s = acc * p.scale;
      }
      ss[idx] = s;
    }
    __syncthreads();
    if (tid < nr) {
      float mx = -INFINITY;
      for (int t = 0; t < kBlock; ++t) mx = fmaxf(mx, ss[tid * kBlock + t]);
      const float m_old = sm[tid];
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, sum = 0.f;
      if (m_new != -INFINITY) {
        alpha = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
        for (int t = 0; t < kBlock; ++t) {
          const float e = expf(ss[tid * kBlock + t] - m_new);
          ss[tid * kBlock + t] = e;
          sum += e;
        }
      }
      sl[tid] = sl[tid] * alpha + sum;
      sm[tid] = m_new;
      sa[tid] = alpha;
    }
    __syncthreads();
    for (int idx = tid; idx < nr * p.dvo; idx += kGenThreads) {
      const int r = idx / p.dvo, f = idx % p.dvo, rr = r0 + r;
      const int n = L - p.s_q + 1 + rr / p.heads_per_kv;
      const int lim = min(kBlock, n - blk * kBlock);   // tokens this row sees in the block
      float acc = so[idx] * sa[r];
      for (int t = 0; t < lim; ++t)
        acc += ss[r * kBlock + t] * Elt<T>::load(base, kv_v_index(p, t, f));
      so[idx] = acc;
    }
    __syncthreads();
  }

  for (int idx = tid; idx < nr * p.dvo; idx += kGenThreads) {
    const int r = idx / p.dvo, f = idx % p.dvo, rr = r0 + r;
    const int i = rr / p.heads_per_kv, h = kvh * p.heads_per_kv + rr % p.heads_per_kv;
    const int64_t row = static_cast<int64_t>(b * p.s_q + i) * p.H + h;
    const float l = sl[r], m = sm[r];
    if (p.n_split == 1) {
      store_out(p.out, p.out_kind, row * p.dvo + f, bad ? nan_f32() : so[idx] / l);
      if (p.lse != nullptr && f == 0) p.lse[row] = bad ? nan_f32() : m + logf(l);
    } else {
      const int64_t slot = row * p.n_split + split;
      p.ws_o[slot * p.dvo + f] = bad ? nan_f32() : (l > 0.f ? so[idx] / l : 0.f);
      if (f == 0) p.ws_lse[slot] = bad ? nan_f32() : (l > 0.f ? m + logf(l) : -INFINITY);
    }
  }
}

hipError_t launch_generic_attn(const AttnParams& p, bool bf16, hipStream_t s) {
  const int rows_total = p.heads_per_kv * p.s_q;
  dim3 grid(p.n_split, (rows_total + kGenRows - 1) / kGenRows, p.B * p.kv_heads);
  const size_t lds = generic_attn_lds_bytes(p.dk, p.dvo);
  hipError_t e;
  if (bf16) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&generic_attn_split<bf16_t>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    generic_attn_split<bf16_t><<<grid, kGenThreads, lds, s>>>(p);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&generic_attn_split<float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    generic_attn_split<float><<<grid, kGenThreads, lds, s>>>(p);
  }
  return hipGetLastError();
}

// Merge split partials: o = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max lse);
// lse = max + ln sum w. A NaN partial (bad metadata) makes the row NaN. Every thread
// derives the weights itself from the row's lse values (L2-resident), then handles four
// consecutive features with 16-byte loads, eight splits at a time: the loads of a batch
// are issued together and an empty split (lse = -inf) is skipped by its weight, not by a
// branch around its load.
constexpr int kMaxCombineSplits = 1024;   // the split plans never exceed this many per row

__global__ __launch_bounds__(128) void combine_splits(CombineParams c) {
  const int64_t row = blockIdx.x;
  const float* lse = c.ws_lse + row * c.n_split;   // re-pointed at LDS on the general path
  constexpr int kFew = 8;
  if ((c.dvo & 3) == 0 && c.n_split <= kFew) {
    // Up to 8 splits: the split lse values and the partial outputs load together (one
    // memory round trip per row instead of two).
    float l[kFew];
#pragma unroll
    for (int s = 0; s < kFew; ++s) l[s] = s < c.n_split ? lse[s] : -INFINITY;
    const float* o = c.ws_o + row * c.n_split * c.dvo;
    for (int f = 4 * threadIdx.x; f < c.dvo; f += 4 * blockDim.x) {
      float4 v[kFew];
#pragma unroll
      for (int s = 0; s < kFew; ++s)
        if (s < c.n_split) v[s] = *reinterpret_cast<const float4*>(o + static_cast<int64_t>(s) * c.dvo + f);
      float m = -INFINITY;
      bool has_nan = false;
#pragma unroll
      for (int s = 0; s < kFew; ++s) {
        has_nan |= l[s] != l[s];
        m = fmaxf(m, l[s]);
      }
      float tot = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int s = 0; s < kFew; ++s) {
        if (s < c.n_split && l[s] != -INFINITY) {
          const float w = expf(l[s] - m);
          tot += w;
          acc.x += w * v[s].x; acc.y += w * v[s].y; acc.z += w * v[s].z; acc.w += w * v[s].w;
        }
      }
      const bool nan_row = has_nan || !(tot > 0.f);
      const float inv = 1.f / tot;
      const float r[4] = {acc.x, acc.y, acc.z, acc.w};
      for (int k = 0; k < 4; ++k) store_out(c.out, c.out_kind, row * c.dvo + f + k, nan_row ? nan_f32() : r[k] * inv);
      if (c.lse != nullptr && f == 0) c.lse[row] = nan_row ? nan_f32() : m + logf(tot);
    }
    return;
  }
  // More splits: the row's lse values are staged in LDS by one parallel load, so the loops
  // over them below do not wait for a memory round trip per split.
  __shared__ float s_lse[kMaxCombineSplits];
  for (int s = threadIdx.x; s < c.n_split; s += blockDim.x) s_lse[s] = lse[s];
  __syncthreads();
  lse = s_lse;
  float m = -INFINITY;
  bool has_nan = false;
  for (int s = 0; s < c.n_split; ++s) {
    const float l = lse[s];
    has_nan |= l != l;
    m = fmaxf(m, l);
  }
  float tot = 0.f;
  for (int s = 0; s < c.n_split; ++s) {
    const float l = lse[s];
    tot += (l == -INFINITY) ? 0.f : expf(l - m);
  }
  const bool nan_row = has_nan || !(tot > 0.f);
  const float inv = 1.f / tot;
  const float* o = c.ws_o + row * c.n_split * c.dvo;
  if ((c.dvo & 3) == 0) {
    constexpr int kBatch = 8;
    for (int f = 4 * threadIdx.x; f < c.dvo; f += 4 * blockDim.x) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s0 = 0; s0 < c.n_split; s0 += kBatch) {
        // Empty slots (lse = -inf: a split past the sequence's end) are not loaded.
        float4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (s0 + j < c.n_split && lse[s0 + j] != -INFINITY)
            v[j] = *reinterpret_cast<const float4*>(o + static_cast<int64_t>(s0 + j) * c.dvo + f);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (s0 + j < c.n_split) {
            const float l = lse[s0 + j];
            if (l != -INFINITY) {
              const float w = expf(l - m);
              acc.x += w * v[j].x; acc.y += w * v[j].y; acc.z += w * v[j].z; acc.w += w * v[j].w;
            }
          }
        }
      }
      const float r[4] = {acc.x, acc.y, acc.z, acc.w};
      for (int k = 0; k < 4; ++k) store_out(c.out, c.out_kind, row * c.dvo + f + k, nan_row ? nan_f32() : r[k] * inv);
    }
  } else {
    for (int f = threadIdx.x; f < c.dvo; f += blockDim.x) {
      float acc = 0.f;
      for (int s = 0; s < c.n_split; ++s) {
        const float l = lse[s];
        if (l == -INFINITY) continue;
        acc += expf(l - m) * o[static_cast<int64_t>(s) * c.dvo + f];
      }
      store_out(c.out, c.out_kind, row * c.dvo + f, nan_row ? nan_f32() : acc * inv);
    }
  }
  if (c.lse != nullptr && threadIdx.x == 0) c.lse[row] = nan_row ? nan_f32() : m + logf(tot);
}

hipError_t launch_combine(const CombineParams& c, hipStream_t s) {
  if (c.n_split > kMaxCombineSplits) return hipErrorInvalidValue;
  combine_splits<<<c.rows, 128, 0, s>>>(c);
  return hipGetLastError();
}

// q_abs[row][h] = [W_UK^g^T q_nope[row][h] ; q_rope[row][h]] (one workgroup per (row, h)).
template <typename T>
__global__ __launch_bounds__(256) void generic_absorb_query(ProjParams d, const T* q_nope, const T* q_rope,
                                                            const T* w_uk, T* q_abs) {
  const int64_t rh = blockIdx.x;             // (b * s_q + i) * H + h
  const int h = static_cast<int>(rh % d.H);
  const int g = h / (d.H / d.G);
  const int dq = d.dc + d.dr;
  for (int c = threadIdx.x; c < dq; c += blockDim.x) {
    float acc;
    if (c < d.dc) {
      acc = 0.f;
      for (int n = 0; n < d.dn; ++n)
        acc += Elt<T>::load(q_nope, rh * d.dn + n) * Elt<T>::load(w_uk, (static_cast<int64_t>(g) * d.dn + n) * d.dc + c);
    } else {
      acc = Elt<T>::load(q_rope, rh * d.dr + (c - d.dc));
    }
    Elt<T>::store(q_abs, rh * dq + c, acc);
  }
}

hipError_t launch_generic_absorb_query(const ProjParams& d, const void* q_nope, const void* q_rope,
                                       const void* w_uk, void* q_abs, bool bf16, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(d.rows) * d.H;
  if (bf16)
    generic_absorb_query<bf16_t><<<n, 256, 0, s>>>(d, static_cast<const bf16_t*>(q_nope), static_cast<const bf16_t*>(q_rope),
                                                 static_cast<const bf16_t*>(w_uk), static_cast<bf16_t*>(q_abs));
  else
    generic_absorb_query<float><<<n, 256, 0, s>>>(d, static_cast<const float*>(q_nope), static_cast<const float*>(q_rope),
                                                static_cast<const float*>(w_uk), static_cast<float*>(q_abs));
  return hipGetLastError();
}

// out[row][h][v] = sum_c W_UV^g[v][c] o_lat[row][h][c]; one wave per output value.
template <typename T>
__global__ __launch_bounds__(256) void generic_out_proj(ProjParams d, const float* o_lat, const T* w_uv, T* out) {
  const int64_t rh = blockIdx.x;
  const int h = static_cast<int>(rh % d.H);
  const int g = h / (d.H / d.G);
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  for (int v = wave; v < d.dv; v += blockDim.x / 64) {
    float acc = 0.f;
    for (int c = lane; c < d.dc; c += 64)
      acc += o_lat[rh * d.dc + c] * Elt<T>::load(w_uv, (static_cast<int64_t>(g) * d.dv + v) * d.dc + c);
    acc = wave_sum(acc);
    if (lane == 0) Elt<T>::store(out, rh * d.dv + v, acc);
  }
}

hipError_t launch_generic_out_proj(const ProjParams& d, const float* o_lat, const void* w_uv,
                                   void* out, bool bf16, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(d.rows) * d.H;
  if (bf16)
    generic_out_proj<bf16_t><<<n, 256, 0, s>>>(d, o_lat, static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(out));
  else
    generic_out_proj<float><<<n, 256, 0, s>>>(d, o_lat, static_cast<const float*>(w_uv), static_cast<float*>(out));
  return hipGetLastError();
}

// Expanded block of id: an optional shared RoPE key area, then per group K in slabs of 32
// features ([64][w_s] each, the last narrower when the feature count is not a multiple of
// 32), then V as two 32-slot halves [d_v][32].
template <typename T>
__global__ __launch_bounds__(256) void generic_expand(ProjParams d, const T* latent, const T* w_uk, const T* w_uv,
                                                      const int32_t* block_ids, int64_t num_blocks, T* expanded) {
  const int32_t id = block_ids[blockIdx.x];
  if (id < 0 || id >= num_blocks) return;
  const int g = blockIdx.y;
  const int dq = d.dc + d.dr, dqk = d.dn + d.dr;
  const ExpandedLayout lay = expanded_layout(d.dn, d.dr, d.dv, d.G, d.rope_shared != 0);
  const T* src = latent + static_cast<int64_t>(id) * kBlock * dq;
  T* blk = expanded + static_cast<int64_t>(id) * lay.block;
  T* dst = blk + lay.rope + g * lay.chunk;
  for (int idx = threadIdx.x; idx < kBlock * dqk; idx += blockDim.x) {
    const int r = idx / dqk, e = idx % dqk;
    float acc;
    if (e < d.dn) {
      acc = 0.f;
      for (int c = 0; c < d.dc; ++c)
        acc += Elt<T>::load(src, static_cast<int64_t>(r) * dq + c) * Elt<T>::load(w_uk, (static_cast<int64_t>(g) * d.dn + e) * d.dc + c);
    } else {
      acc = Elt<T>::load(src, static_cast<int64_t>(r) * dq + d.dc + (e - d.dn));
    }
    if (e < lay.k_feats) {
      const int s = e / kSlab, w = min(kSlab, lay.k_feats - s * kSlab);
      Elt<T>::store(dst, static_cast<int64_t>(s) * kBlock * kSlab + r * w + (e - s * kSlab), acc);
    } else if (g == 0) {   // shared RoPE key, written once per block
      const int f = e - d.dn, s = f / kSlab, w = min(kSlab, d.dr - s * kSlab);
      Elt<T>::store(blk, static_cast<int64_t>(s) * kBlock * kSlab + r * w + (f - s * kSlab), acc);
    }
  }
  for (int idx = threadIdx.x; idx < d.dv * kBlock; idx += blockDim.x) {
    const int f = idx / kBlock, r = idx % kBlock;
    float acc = 0.f;
    for (int c = 0; c < d.dc; ++c)
      acc += Elt<T>::load(src, static_cast<int64_t>(r) * dq + c) * Elt<T>::load(w_uv, (static_cast<int64_t>(g) * d.dv + f) * d.dc + c);
    Elt<T>::store(dst, static_cast<int64_t>(kBlock) * lay.k_feats + (r / kHalf) * d.dv * kHalf + f * kHalf + r % kHalf, acc);
  }
}

hipError_t launch_generic_expand(const ProjParams& d, const void* latent, const void* w_uk,
                                 const void* w_uv, const int32_t* block_ids, int64_t n_blocks,
                                 int64_t num_blocks, void* expanded, bool bf16, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(n_blocks), d.G);
  if (bf16)
    generic_expand<bf16_t><<<grid, 256, 0, s>>>(d, static_cast<const bf16_t*>(latent), static_cast<const bf16_t*>(w_uk),
                                               static_cast<const bf16_t*>(w_uv), block_ids, num_blocks, static_cast<bf16_t*>(expanded));
  else
    generic_expand<float><<<grid, 256, 0, s>>>(d, static_cast<const float*>(latent), static_cast<const float*>(w_uk),
                                              static_cast<const float*>(w_uv), block_ids, num_blocks, static_cast<float*>(expanded));
  return hipGetLastError();
}

}  // namespace gqla
