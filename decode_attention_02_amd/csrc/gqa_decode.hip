// GQA-path split-KV decode on gfx950 MFMA (bf16 data, fp32 accumulation).
//
// Grouped-query attention over the per-group expanded cache: the gs query heads of a
// group share one key head and one value head ("Grouped Query Attention (GQA)", section
// "Fonctionnement de la GQA"), and GQLA's GQA path runs exactly that over the latent
// expanded into G key/value heads ("GQLA: Attention latente ...", English abstract).
//
// Decode is bound by reading the cache ("Pourquoi la GQA réduit le cache KV"), so the
// kernel is built around streaming each (block, group) chunk of 64 tokens x
// (d_qk + d_v) bf16 exactly once, with 128-bit loads straight into MFMA operand
// registers:
//   * one workgroup = (sequence, group, split); its waves take interleaved 64-token
//     blocks of the split and keep private online-softmax states, merged in LDS at
//     the end; when sequences x groups do not cover the CUs, a workgroup instead takes
//     one of the equal runs of the batch's blocks laid end to end (attend_balanced);
//   * scores are formed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16, A = 16
//     tokens x 32 features of K, B = 32 features x 16 query rows), so each lane owns
//     one query row: its running max/sum need only two cross-lane shuffles per step;
//   * K rows are gathered in a permuted token order so that each lane ends up holding
//     8 consecutive tokens, which is exactly the B-operand slice of P^T for the value
//     product O^T = V^T P^T; V is stored feature-major (per 32-token half), so its A
//     operand is again one 128-bit load per lane and P never leaves registers.
// Rows: query row j < gs * s_q of a group is (i = j / gs, head = g * gs + j % gs);
// rows beyond gs * s_q (up to the 16 of an MFMA tile) carry zero queries.
#include "device_common.h"
#include "gqla_internal.h"
#include "balanced_plan.h"
#include "tuned.h"

#include <cmath>

namespace gqla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// Cache operands are read exactly once, each load covering whole 128-byte lines (the
// expanded cache's slab layout), so they bypass cache retention.
__device__ __forceinline__ bf16x8 load8_stream(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p)));
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// RT = 16-row MFMA column tiles of query rows per group (gs * s_q <= 16 * RT); with two,
// every K and V operand load feeds both tiles. SHARED: the expanded cache keeps the RoPE
// key (d_R = 64) once per block; its K slabs come from the block's key area, and the
// workgroups of one sequence's groups are placed on one XCD so that area is fetched from
// HBM once and served to the other groups from that XCD's L2.
template <int DQK, int DV, int kWaves, int RT, bool SHARED>
__device__ __forceinline__ void attend(const AttnParams& p, int b, int g, int blk_lo, int blk_end, int slot,
                                       int limit_blocks) {
  constexpr int KS = DQK / 32;     // k-steps of the score product
  constexpr int KSN = SHARED ? (DQK - 64) / 32 : KS;   // k-steps held in the group chunk
  constexpr int KF = 32 * KSN;     // K features in the group chunk
  constexpr int NT = DV / 16;      // feature tiles of the value product
  constexpr bool kHalfUnits = (RT == 2 && DQK > 128) || RT == 1;
  __shared__ float s_o[kWaves][RT][NT][64][4];   // per-wave O^T fragments (lane-major)
  __shared__ float s_m[kWaves][RT * 16];
  __shared__ float s_l[kWaves][RT * 16];
  __shared__ int s_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;          // query row owned by this lane in each tile (MFMA column)
  const int grp = lane >> 4;          // k-group of the MFMA operands
  const int gs = p.heads_per_kv;
  const int rows = gs * p.s_q;

  const int L = p.ctx_lens[b];
  const int nblk = (L + kBlock - 1) / kBlock;
  bool bad = (L < p.s_q) || (L > p.max_blocks * kBlock) || (nblk > limit_blocks);

  // This lane's query rows (one per tile) and their visible-token limits; B operand of S^T:
  // Q^T slices (features 32*ks + 8*grp .. +8 of query row 16*r + col).
  int n_vis[RT];
  bf16x8 qf[RT][KS];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int j = 16 * r + col;
    const int qi = j / gs;
    const int qh = g * gs + j % gs;
    const bool live_row = j < rows;
    n_vis[r] = live_row ? L - p.s_q + 1 + qi : L;
    const bf16_t* q = static_cast<const bf16_t*>(p.q) +
                      (static_cast<int64_t>(b * p.s_q + qi) * p.H + qh) * DQK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (live_row) qf[r][ks] = load8(q + 32 * ks);
      else qf[r][ks] = bf16x8{};
    }
  }

  f32x4 acc[RT][NT];
  float m_run[RT], l_run[RT];   // running max (log2 domain) and this lane's running sum
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[r][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  const float qk_scale = p.scale * kLog2e;

  const bf16_t* kv = static_cast<const bf16_t*>(p.kv);
  const int32_t* table = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int blk_hi = bad ? blk_lo : min(nblk, blk_end);
  // This wave's blocks: first, first + kWaves, ... (n_my of them).
  const int first = blk_lo + wave;
  const int n_my = blk_hi > first ? (blk_hi - first + kWaves - 1) / kWaves : 0;

  // Block ids, 64 at a time: lane i holds the id of this wave's block 64*c + i. An id
  // outside the pool marks the whole row bad and is replaced by 0 so loads stay in bounds.
  int ids = 0, ids_chunk = -1;
  auto block_id = [&](int j) -> int {
    const int c = j >> 6;
    if (c != ids_chunk) {
      const int jj = 64 * c + lane;
      const int v = jj < n_my ? table[first + kWaves * jj] : 0;
      const bool inval = jj < n_my && (v < 0 || v >= p.num_blocks);
      bad |= __ballot(inval) != 0;
      ids = inval ? 0 : v;
      ids_chunk = c;
    }
    return __builtin_amdgcn_readlane(ids, j & 63);
  };
  auto chunk_of = [&](int id) -> const bf16_t* {
    return kv + static_cast<int64_t>(id) * p.block_stride + p.kv_off + g * p.kvh_stride;
  };

  // One half block's operands: K rows of its 32 tokens, permuted so lane group `grp`
  // gets tokens 32*half + 8*grp .. +8, and V^T slices of the same tokens. K features
  // 32*ks .. +32 of all 64 tokens form one slab ([64][32]), V^T is stored as two 32-token
  // halves ([DV][32]): each load instruction reads four 256-byte runs of K or one 1 KiB
  // run of V^T.
  struct Half {
    bf16x8 k[2][KS];
    bf16x8 v[NT];
  };
  auto load_half = [&](Half& f, const bf16_t* chunk, int half) {
    const bf16_t* vt = chunk + kBlock * KF;
    const bf16_t* rk = chunk - (p.kv_off + g * p.kvh_stride);   // the block's shared key area
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 32 * half + 8 * (col >> 2) + 4 * tt + (col & 3);
      const bf16_t* krow = chunk + tok * kSlab + 8 * grp;
      const bf16_t* rrow = rk + tok * kSlab + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        f.k[tt][ks] = ks < KSN ? load8_stream(krow + ks * kBlock * kSlab)
                               : load8(rrow + (ks - KSN) * kBlock * kSlab);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      f.v[nt] = load8_stream(vt + half * DV * kHalf + (16 * nt + col) * kHalf + 8 * grp);
  };

  auto compute_half = [&](const Half& f, int blk, int half) {
    f32x4 s[RT][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < RT; ++r) s[r][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          s[r][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[tt][ks], qf[r][ks], s[r][tt], 0, 0, 0);
    }
    // Token of score s[r][tt][k] in this lane: blk*64 + 32*half + 8*grp + 4*tt + k.
    const int tbase = blk * kBlock + 32 * half + 8 * grp;
    bf16x8 pf[RT];
    float alpha[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = (tbase + 4 * tt + k < n_vis[r]) ? s[r][tt][k] * qk_scale : -INFINITY;
          sc[4 * tt + k] = v;
          mx = fmaxf(mx, v);
        }
      mx = xor_max(mx);
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[r] = __builtin_amdgcn_exp2f(m_run[r] - m_use);
      m_run[r] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float e = __builtin_amdgcn_exp2f(sc[k] - m_use);
        psum += e;
        pf[r][k] = static_cast<__bf16>(e);
      }
      l_run[r] = l_run[r] * alpha[r] + psum;
    }
    // Slots past the context hold arbitrary bits (possibly NaN): their value columns
    // are masked to zero, two tokens per 32-bit word.
    u32x4 keep = {~0u, ~0u, ~0u, ~0u};
    if (blk * kBlock + kBlock > L) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        keep[w] = (tbase + 2 * w < L ? 0xffffu : 0u) | (tbase + 2 * w + 1 < L ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 vm = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f.v[nt]) & keep);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        acc[r][nt] *= alpha[r];
        acc[r][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vm, pf[r], acc[r][nt], 0, 0, 0);
      }
    }
  };

  if constexpr (!kHalfUnits) {
    // Two blocks in flight per wave: the next block's loads are issued before the current
    // one is consumed. Past the last block the last one is fetched again (an L2 hit), so
    // every iteration issues the same loads and the waits stay exact.
    auto load = [&](Half (&f)[2], const bf16_t* chunk) { load_half(f[0], chunk, 0); load_half(f[1], chunk, 1); };
    auto compute = [&](const Half (&f)[2], int blk) { compute_half(f[0], blk, 0); compute_half(f[1], blk, 1); };
    if (n_my > 0) {
      Half fa[2], fb[2];
      load(fa, chunk_of(block_id(0)));
      for (int j = 0; j < n_my; j += 2) {
        load(fb, chunk_of(block_id(min(j + 1, n_my - 1))));
        __builtin_amdgcn_sched_barrier(0);
        compute(fa, first + kWaves * j);
        load(fa, chunk_of(block_id(min(j + 2, n_my - 1))));
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < n_my) compute(fb, first + kWaves * (j + 1));
      }
    }
  } else {
    // Two half blocks in flight (the next half's loads issued before the current half is
    // consumed): the register budget of two row tiles at d_qk = 192, and of two workgroups
    // per CU (two waves per SIMD) with one row tile.
    if (n_my > 0) {
      const int nu = 2 * n_my;
      auto unit_chunk = [&](int u) { return chunk_of(block_id(min(u, nu - 1) >> 1)); };
      Half fa, fb;
      load_half(fa, unit_chunk(0), 0);
      for (int u = 0; u < nu; u += 2) {
        load_half(fb, unit_chunk(u + 1), 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(fa, first + kWaves * (u >> 1), 0);
        load_half(fa, unit_chunk(u + 2), min(u + 2, nu - 1) & 1 ? 1 : 0);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(fb, first + kWaves * (u >> 1), 1);
      }
    }
  }

  // Merge the waves: O = sum_w 2^(m_w - M) O_w, l = sum_w 2^(m_w - M) l_w.
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    l_run[r] = xor_sum(l_run[r]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(&s_o[wave][r][nt][lane][0]) = acc[r][nt];
    if (grp == 0) { s_m[wave][16 * r + col] = m_run[r]; s_l[wave][16 * r + col] = l_run[r]; }
  }
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();
  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= s_bad[w] != 0;
  // Thread -> (query row jr, 8 consecutive features), 16 threads per row.
  for (int item = threadIdx.x; item < 16 * RT * (DV / 8); item += kWaves * 64) {
    const int jr = item / (DV / 8);
    const int f0 = (item % (DV / 8)) * 8;
    if (jr >= rows) break;   // items are row-major, so every later one is past the rows too
    const int r = jr >> 4, c = jr & 15;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][jr]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float wgt[kWaves];
    float l_tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = __builtin_amdgcn_exp2f(s_m[w][jr] - M_use);
      l_tot += wgt[w] * s_l[w][jr];
    }
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // feature f = f0 + k lives in tile f/16, lane (c + 16 * ((f % 16) / 4)), slot f % 4
      const int f = f0 + k;
      const int ln = c + 16 * ((f & 15) >> 2);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += wgt[w] * s_o[w][r][f >> 4][ln][f & 3];
      o[k] = v;
    }
    const int i = jr / gs;
    const int h = g * gs + jr % gs;
    const int64_t row = static_cast<int64_t>(b * p.s_q + i) * p.H + h;
    if (p.n_split == 1) {
      const float inv = 1.f / l_tot;
      bf16_t packed[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) packed[k] = any_bad ? 0x7fc0 : f32_to_bf16(o[k] * inv);
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(p.out) + row * DV + f0) = *reinterpret_cast<uint4*>(packed);
      if (p.lse != nullptr && f0 == 0) p.lse[row] = any_bad ? nan_f32() : (M + __log2f(l_tot)) * kLn2;
    } else {
      const int64_t at = row * p.n_split + slot;
      const bool empty = !(l_tot > 0.f);
      float* dst = p.ws_o + at * DV + f0;
#pragma unroll
      for (int k = 0; k < 8; k += 4) {
        f32x4 v;
        for (int u = 0; u < 4; ++u) v[u] = any_bad ? nan_f32() : (empty ? 0.f : o[k + u] / l_tot);
        *reinterpret_cast<f32x4*>(dst + k) = v;
      }
      if (f0 == 0) p.ws_lse[at] = any_bad ? nan_f32() : (empty ? -INFINITY : (M + __log2f(l_tot)) * kLn2);
    }
  }
}

// Length-balanced plan (balanced_plan.h): run c of group g attends to each piece of the
// sequences it meets in turn, then marks a finished sequence's unused slots empty.
template <int DQK, int DV, int kWaves, int RT, bool SHARED>
__device__ __forceinline__ void attend_balanced(const AttnParams& p, int c, int g) {
  const BalancedRun run = balanced_run(p, c);
  if (run.empty) return;
  const int C = run.C, lo = run.lo, hi = run.hi;
  const int gs = p.heads_per_kv;
  const int rows = gs * p.s_q;
  int e = run.start;
  for (int b = run.b; b < p.B; ++b) {
    const int s0 = e;
    e += plan_blocks(p, b);
    if (s0 >= hi) break;
    if (b != run.b) __syncthreads();   // the previous piece's merge has read the LDS
    attend<DQK, DV, kWaves, RT, SHARED>(p, b, g, max(lo, s0) - s0, min(hi, e) - s0, c - s0 / C, p.decl_blocks);
    if (e <= hi) {
      const int used = (e - 1) / C - s0 / C + 1;
      for (int item = threadIdx.x; item < rows * (p.n_split - used); item += kWaves * 64) {
        const int jr = item % rows, sl = used + item / rows;
        const int64_t row = static_cast<int64_t>(b * p.s_q + jr / gs) * p.H + g * gs + jr % gs;
        p.ws_lse[row * p.n_split + sl] = -INFINITY;
      }
    }
  }
}

// BAL: the length-balanced plan (its own instantiation, so the planning code does not
// change the register allocation of the streaming loop in the other one).
template <int DQK, int DV, int kWaves, int RT, bool SHARED, bool BAL>
__global__ __launch_bounds__(kWaves * 64, RT == 1 ? 2 : 1) void gqa_decode_split(AttnParams p) {
  const int units = BAL ? p.chunks : p.B * p.n_split;
  int u, g;
  if constexpr (SHARED) {
    // id = ((u / 8) * G + g) * 8 + u % 8 for unit u = (sequence, split) or balanced run: a
    // unit's groups share an XCD (ids equal mod 8) and are dispatched together.
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    g = y % p.kv_heads;
    u = (y / p.kv_heads) * 8 + x;
    if (u >= units) return;
  } else if constexpr (BAL) {
    u = blockIdx.x % units;
    g = blockIdx.x / units;
  } else {
    const int split = blockIdx.x % p.n_split, bg = blockIdx.x / p.n_split;
    g = bg % p.kv_heads;
    u = (bg / p.kv_heads) * p.n_split + split;
  }
  if constexpr (BAL) {
    attend_balanced<DQK, DV, kWaves, RT, SHARED>(p, u, g);
  } else {
    const int split = u % p.n_split, b = u / p.n_split;
    const int blk_lo = split * p.blocks_per_split;
    attend<DQK, DV, kWaves, RT, SHARED>(p, b, g, blk_lo, blk_lo + p.blocks_per_split, split,
                                        p.n_split * p.blocks_per_split);
  }
}

}  // namespace

bool tuned_gqa_supported(const gqla_dims* d) {
  const int dqk = d->nope_dim + d->rope_dim;
  const int gs = d->num_heads / d->num_groups;
  return d->dtype == GQLA_BF16 && (dqk == 128 || dqk == 192) && d->v_dim == 128 && gs * d->s_q <= 32 &&
         (d->rope_shared == 0 || d->rope_dim == 64);
}

// One workgroup per CU per round: on MI355X the unsplit launch streams fastest
// (LLaMA-3-8B batch 32 s_q = 2, shared RoPE key: 129 us unsplit against 139 / 153 us with
// two / four splits and a combine),
// so the context is only split when sequences x groups cannot cover the CUs.
int tuned_gqa_target_wgs() { return kNumCUs; }
int tuned_gqa_min_blocks_per_split() { return 8; }

// Four waves per workgroup. With one row tile each wave keeps half a block in flight within
// 256 registers, so two workgroups share a CU (two waves per SIMD): one wave's loads run while
// the other does its softmax, and one workgroup streams while the other starts (block ids,
// queries, first block) or merges its waves. Against one 8-wave workgroup per CU with the same
// per-wave code: LLaMA-3-8B batch 32 131.5 -> 126.8 us, DeepSeek-V3 batch 64 675 -> 655 us,
// the long-context batch equal, the 1/8 DeepSeek-V3 share 29.14 -> 28.99 ms. Two row tiles
// need the registers of one wave per SIMD.
template <int DQK, int RT, bool SHARED>
hipError_t launch_dqk(const AttnParams& p, hipStream_t s) {
  constexpr int kWaves = 4;
  const int64_t units = p.chunks > 0 ? p.chunks : static_cast<int64_t>(p.B) * p.n_split;
  const int64_t wgs = SHARED ? (units + 7) / 8 * 8 * p.kv_heads : units * p.kv_heads;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (p.chunks > 0)
    gqa_decode_split<DQK, 128, kWaves, RT, SHARED, true><<<static_cast<unsigned>(wgs), kWaves * 64, 0, s>>>(p);
  else
    gqa_decode_split<DQK, 128, kWaves, RT, SHARED, false><<<static_cast<unsigned>(wgs), kWaves * 64, 0, s>>>(p);
  return hipGetLastError();
}

template <bool SHARED>
hipError_t launch_layout(const AttnParams& p, const gqla_dims* d, hipStream_t s) {
  const bool two = p.heads_per_kv * p.s_q > 16;
  if (d->nope_dim + d->rope_dim == 192) return two ? launch_dqk<192, 2, SHARED>(p, s) : launch_dqk<192, 1, SHARED>(p, s);
  return two ? launch_dqk<128, 2, SHARED>(p, s) : launch_dqk<128, 1, SHARED>(p, s);
}

hipError_t launch_tuned_gqa(const AttnParams& p, const gqla_dims* d, hipStream_t s) {
  return d->rope_shared ? launch_layout<true>(p, d, s) : launch_layout<false>(p, d, s);
}

}  // namespace gqla
