// MQA-absorb split-KV decode on gfx950 MFMA (bf16 latent, fp32 accumulation).
//
// Every query head, with W_UK^g folded into it, attends over the one shared latent
// "key head" [c_KV | k_rope] and takes the latent c_KV itself as its value (MLA's
// absorbed form, which GQLA keeps unchanged: "GQLA: Attention latente ...", English
// abstract; gqla_attn.py docstring: a single MQA-style head per layer).
//
// All H * s_q query rows of a sequence read the same 64-token latent tiles, so the
// tile is fetched from HBM once per workgroup and shared through LDS:
//   * tiles (64 tokens x 576 bf16 = 72 KiB) are copied global -> LDS by
//     global_load_lds_dwordx4 (no register staging), double-buffered, with an XOR
//     swizzle of the 16-byte chunks inside each 128-byte group so that both LDS
//     access patterns below are bank-conflict free;
//   * each wave owns 16 query rows (one MFMA tile): scores S^T = C Q^T
//     (v_mfma_f32_16x16x32_bf16, A = 16 tokens x 32 latent features read with
//     ds_read_b128, B = the wave's absorbed queries held in registers);
//   * the value product O^T = C^T P^T needs the latent with tokens along the
//     contraction, which ds_read_b64_tr_b16 delivers directly from the row-major tile;
//     P stays in registers as the B operand;
//   * small row counts (16 or 32 rows) also split each tile's two 32-token halves
//     over two waves, merged at the end, so a workgroup still has 4 waves streaming;
//   * more than 128 rows use two workgroups per (sequence, split), placed on the same
//     XCD so the second tile read is served from that XCD's L2;
//   * from 64 rows on, waves work in feature-split pairs (AbsorbPairCta): each wave
//     scores its own 16 rows, the pair swaps P through LDS, and each wave's transposed
//     value reads then serve both tiles for half of the latent features.
#include "device_common.h"
#include "gqla_internal.h"
#include "tuned.h"

#include <cmath>

namespace gqla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDC = 512;                 // latent rank
constexpr int kDQ = 576;                 // latent + RoPE values per token
constexpr int kRowBytes = kDQ * 2;       // 1152
constexpr int kChunks = kDQ / 8;         // 16-byte chunks per token row (72)
constexpr int kTileBytes = kBlock * kRowBytes;  // 73728
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Swizzle of a token row's 16-byte chunk index inside its 128-byte group. gfx950's LDS
// serves 256 bytes per cycle and a 1152-byte row stride alternates rows between the two
// 128-byte halves, so conflict-free access needs, for the score reads (16 rows, one
// chunk each), distinct (t & 1, swz) over 16 consecutive rows, and for the transposed
// reads (8 rows, a chunk pair each), distinct swz >> 1 among same-parity rows of each
// aligned 8: swz(t) = (t mod 8) xor bit 3 of t satisfies both and has period 16.
__device__ __forceinline__ int swz(int t) { return (t & 7) ^ ((t >> 3) & 1); }
__device__ __forceinline__ int chunk_off(int t, int c) {
  return t * kRowBytes + (((c & ~7) | ((c & 7) ^ swz(t))) << 4);
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low bits [3:0], high
// bits [15:14]; expcnt and lgkmcnt fields left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ void lds_barrier() {
  // Workgroup barrier without the memory fence of __syncthreads(): the fence would
  // also wait for the next tile's copy, which must stay in flight. Callers wait for
  // exactly the counters they need first.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane l's bytes
// land at lds + 16 * l.
__device__ __forceinline__ void copy16_to_lds(const char* g, lds_void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 2);
}

constexpr int kMaxSplitBlocks = 1024;    // block ids of one split staged in LDS
constexpr float kRescaleSlack = 8.f;     // log2 headroom before the accumulator is rescaled
constexpr int kScoreBatch = 6;           // score operand reads per batch (36 per 32 tokens)
constexpr int kValueBatch = 4;           // value feature tiles per batch (2 reads each)

// The two tile buffers are distinct LDS objects so that the compiler can see that a
// copy into one never aliases reads of the other, and keeps the copy in flight.
__shared__ __attribute__((aligned(16))) char g_tile0[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_tile1[kTileBytes];
__shared__ int32_t g_ids[kMaxSplitBlocks];

template <int BUF>
__device__ __forceinline__ char* tile_buf() { return BUF == 0 ? g_tile0 : g_tile1; }

// Byte offset, inside a block, of the chunk that lands in LDS slot `slot` of a tile.
__device__ __forceinline__ int slot_source(int slot) {
  const int t = slot / kChunks, cp = slot - t * kChunks;
  return t * kRowBytes + 16 * ((cp & ~7) | ((cp & 7) ^ swz(t)));
}

// RPW = 16-row tiles per wave (1 or 2; two tiles share every LDS operand read),
// RT = row tiles per workgroup, TG = waves splitting each tile's two 32-token halves.
template <int RPW, int RT, int TG>
struct AbsorbCta {
  static constexpr int WR = RT / RPW;                          // waves along rows
  static constexpr int W = WR * TG;
  static constexpr int PER_WAVE = kChunks * kBlock / 64 / W;   // 1 KiB copies per wave per tile
  static_assert(PER_WAVE * W * 64 == kChunks * kBlock, "tile must split evenly over waves");
  // Each wave copies whole 16-row periods of the swizzle, so its copy pattern is the same
  // lane pattern at a wave-uniform (scalar) offset.
  static_assert((PER_WAVE * 64) % (16 * kChunks) == 0, "wave copy block must hold whole swizzle periods");
  static constexpr int FT = kDC / 16;                          // feature tiles of O^T
  static constexpr int KS = kDQ / 32;                          // k-steps of the score product

  const AttnParams& p;
  int lane, wave, wr, tg, col, grp;
  int b, split, L, blk_lo, nb;
  bool bad;
  int qi[RPW], qh[RPW], n_vis[RPW];
  bf16x8 qf[RPW][KS];
  f32x4 acc[RPW][FT];
  float m_ref[RPW], l_run[RPW];
  float qk_scale;
  // per-lane LDS byte offsets (see score() and value())
  int s_base_even, s_base_odd;
  int v_base[4];
  uint32_t dma_off[PER_WAVE];   // per-lane source offsets of the tile copy, within the wave's rows

  __device__ AbsorbCta(const AttnParams& p_) : p(p_) {}

  // Copy of the tile of the k-th block of the split into buffer BUF. Wave instruction j
  // writes LDS slots (wave * PER_WAVE + j) * 64 + lane, each a 16-byte chunk; the lane
  // fetches the logical chunk that the swizzle stores at its slot.
  __device__ __forceinline__ const char* tile_src(int k) const {
    const int32_t id = max(g_ids[k], 0);   // invalid ids already poisoned the output
    return static_cast<const char*>(p.kv) + static_cast<int64_t>(id) * kTileBytes + wave * PER_WAVE * 1024;
  }
  template <int BUF, int J>
  __device__ __forceinline__ void issue_one(const char* src) {
    copy16_to_lds(src + dma_off[J], (lds_void*)(tile_buf<BUF>() + (wave * PER_WAVE + J) * 1024));
  }
  template <int BUF, int J = 0>
  __device__ __forceinline__ void issue_all(const char* src) {
    if constexpr (J < PER_WAVE) {
      issue_one<BUF, J>(src);
      issue_all<BUF, J + 1>(src);
    }
  }


  // Slots past the context in the last block hold arbitrary bits: zero those token rows
  // in LDS once, so the value product needs no per-element masking.
  template <int BUF>
  __device__ __forceinline__ void clear_tail(int valid) {
    char* tile = tile_buf<BUF>();
    for (int i = valid * kChunks + threadIdx.x; i < kBlock * kChunks; i += W * 64)
      *reinterpret_cast<uint4*>(tile + 16 * i) = uint4{0u, 0u, 0u, 0u};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
  }

  // Scores S^T = C Q^T of the 32 tokens t0 .. t0+31 for each row tile of the wave.
  // Chunk 4*ks + grp of token row `tok` sits at tok*1152 + 16*(...) per the swizzle;
  // since tok = t0 + 16*tt + col with t0 + 16*tt a multiple of 8, swz(tok) = swz(col)
  // and the address is a per-lane base (even or odd ks) plus a compile-time offset.
  // The two 16-token tiles are independent MFMA chains, interleaved. Operand reads go
  // in batches: batch k + 1 is issued right after the first MFMA of batch k, so the
  // single wait per batch (the compiler drains the LDS counter completely while tile
  // copies into LDS are in flight) finds its data already landed.
  // Copies J0 .. J0+CNT-1 of the next tile (into the other buffer, when `nxt` is set) ride
  // along, one after every (2 * KS) / CNT MFMAs, so the copy stream never stalls the wave
  // for long and keeps running while it computes.
  template <int BUF, int J0, int CNT>
  __device__ __forceinline__ void score(int t0, f32x4 (&s)[RPW][2], const char* nxt) {
    const char* tile = tile_buf<BUF>() + t0 * kRowBytes;
    constexpr int N = 2 * KS;   // operand i = (ks = i / 2, tt = i % 2)
    constexpr int D = kScoreBatch;
    static_assert(N % D == 0, "score batches");
    auto ld = [&](int i) {
      const int ks = i >> 1, tt = i & 1;
      return *reinterpret_cast<const bf16x8*>(tile + tt * 16 * kRowBytes + ((ks & 1) ? s_base_odd : s_base_even) +
                                              128 * (ks >> 1));
    };
#pragma unroll
    for (int r = 0; r < RPW; ++r) s[r][0] = s[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a[N];
#pragma unroll
    for (int i = 0; i < D; ++i) a[i] = ld(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        s[r][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], qf[r][i >> 1], s[r][i & 1], 0, 0, 0);
      if (i % D == 0 && i + D < N) {
#pragma unroll
        for (int j = 0; j < D; ++j) a[i + D + j] = ld(i + D + j);
      }
      constexpr int GAP = N / CNT;
      if constexpr (CNT > 0) {
        if (i % GAP == GAP - 1 && i / GAP < CNT && nxt != nullptr) copy_at<1 - BUF, J0>(i / GAP, nxt);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Copy J0 + j (j runtime but in [0, CNT), resolved by a compile-time switch).
  template <int BUF, int J0, int J = J0>
  __device__ __forceinline__ void copy_at(int j, const char* src) {
    if constexpr (J < PER_WAVE) {
      if (j == J - J0) issue_one<BUF, J>(src);
      else copy_at<BUF, J0, J + 1>(j, src);
    }
  }

  // O^T += C^T P^T over the 32 tokens t0 .. t0+31: lane (feature f, group grp) needs the
  // latent of tokens t0 + 4*grp + {0..3} and t0 + 16 + 4*grp + {0..3}; each 16-lane group
  // feeds ds_read_b64_tr_b16 with 4 features 4*(col&3) of token row col>>2. Per-lane
  // bases exist for the four values of ft & 3; the rest is a compile-time offset. The
  // transposed reads are batched like the score operands.
  template <int BUF>
  __device__ __forceinline__ void value(int t0, const bf16x8 (&pf)[RPW]) {
    const char* tile = tile_buf<BUF>() + t0 * kRowBytes;
    constexpr int D = kValueBatch;
    static_assert(FT % D == 0, "value batches");
    auto tr = [&](int ft, int second) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(tile + v_base[ft & 3] + 128 * (ft >> 2) + second * 16 * kRowBytes));
    };
    i16x4 lo[FT], hi[FT];
#pragma unroll
    for (int ft = 0; ft < D; ++ft) { lo[ft] = tr(ft, 0); hi[ft] = tr(ft, 1); }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const i16x8 av = __builtin_shufflevector(lo[ft], hi[ft], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        acc[r][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pf[r], acc[r][ft], 0, 0, 0);
      if (ft % D == 0 && ft + D < FT) {
#pragma unroll
        for (int j = 0; j < D; ++j) { lo[ft + D + j] = tr(ft + D + j, 0); hi[ft + D + j] = tr(ft + D + j, 1); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Online softmax of one 32-token step for row tile r; returns P^T as the B operand.
  __device__ __forceinline__ bf16x8 softmax(int r, const f32x4 (&sr)[2], int tb) {
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const float v = (tb + 16 * tt + k2 < n_vis[r]) ? sr[tt][k2] * qk_scale : -INFINITY;
        sc[4 * tt + k2] = v;
        mx = fmaxf(mx, v);
      }
    mx = xor_max(mx);
    const bool grow = mx > m_ref[r] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform, rare after the first block
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref[r] - mx) : 1.f;
      if (grow) m_ref[r] = mx;
      l_run[r] *= alpha;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) acc[r][ft] *= alpha;
    }
    const float m_use = (m_ref[r] == -INFINITY) ? 0.f : m_ref[r];
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = __builtin_amdgcn_exp2f(sc[j] - m_use);
      psum += e;
      pf[j] = static_cast<__bf16>(e);
    }
    l_run[r] += psum;
    return pf;
  }

  // One 64-token block slot held in buffer BUF (k-th block of the split): wait for its
  // copy, then compute it while the copy of block k + 1 into the other buffer is issued
  // piecemeal from inside the score loop. The other buffer is free: every wave has passed
  // this step's opening barrier, so all of them are done reading it.
  template <int BUF>
  __device__ __forceinline__ void step(int k) {
    __builtin_amdgcn_s_waitcnt(0);   // this block's copy has landed, this wave's LDS reads are done
    lds_barrier();
    if (k < nb) {
      const int blk = blk_lo + k;
      const char* nxt = k + 1 < nb ? tile_src(k + 1) : nullptr;
      if ((blk + 1) * kBlock > L) clear_tail<BUF>(L - blk * kBlock);
      if constexpr (TG == 2) {
        half_step<BUF, 0, PER_WAVE>(tg, blk, nxt);
      } else {
        static_assert(PER_WAVE % 2 == 0, "copies split over the two halves");
        half_step<BUF, 0, PER_WAVE / 2>(0, blk, nxt);
        half_step<BUF, PER_WAVE / 2, PER_WAVE / 2>(1, blk, nxt);
      }
    }
    // No closing barrier: the next step's opening barrier is passed only once every wave
    // has finished this one, and the copy into this buffer is issued after it.
  }

  template <int BUF, int J0, int CNT>
  __device__ __forceinline__ void half_step(int hh, int blk, const char* nxt) {
    const int t0 = hh * 32;
    f32x4 s[RPW][2];
    score<BUF, J0, CNT>(t0, s, nxt);
    const int tb = blk * kBlock + t0 + 4 * grp;
    bf16x8 pf[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) pf[r] = softmax(r, s[r], tb);
    value<BUF>(t0, pf);
  }

  __device__ __forceinline__ void run(int unit, int part) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wr = wave % WR;
    tg = wave / WR;
    col = lane & 15;
    grp = lane >> 4;
    split = unit % p.n_split;
    b = unit / p.n_split;
    L = p.ctx_lens[b];
    const int nblk = (L + kBlock - 1) / kBlock;
    bad = (L < p.s_q) || (L > p.max_blocks * kBlock) || (nblk > p.n_split * p.blocks_per_split);
    blk_lo = split * p.blocks_per_split;
    const int blk_hi = bad ? blk_lo : min(nblk, blk_lo + p.blocks_per_split);
    nb = max(0, blk_hi - blk_lo);

    // The first tile's copy starts before the rest of the prologue; the block ids (staged
    // in LDS, -1 marking an id outside the pool) and the queries load while it runs.
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dma_off[j] = slot_source(j * 64 + lane);
    const int32_t* table = p.block_table + static_cast<int64_t>(b) * p.max_blocks + blk_lo;
    if (nb > 0) {
      const int32_t id0 = table[0];
      const int32_t c0 = (id0 < 0 || id0 >= p.num_blocks) ? 0 : id0;   // a bad id poisons the output anyway
      issue_all<0>(static_cast<const char*>(p.kv) + static_cast<int64_t>(c0) * kTileBytes + wave * PER_WAVE * 1024);
    }
    constexpr int kIdsPerThread = kMaxSplitBlocks / (W * 64);
    int32_t idr[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      idr[u] = i < nb ? table[i] : 0;
    }

    // Rows of this lane, one per row tile r: row = (part * RT + wr * RPW + r) * 16 + col,
    // i.e. query row i = row / H of head h = row % H.
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = (part * RT + wr * RPW + r) * 16 + col;
      qi[r] = row / p.H;
      qh[r] = row % p.H;
      n_vis[r] = L - p.s_q + 1 + qi[r];
      const bf16_t* q = static_cast<const bf16_t*>(p.q) +
                        (static_cast<int64_t>(b * p.s_q + qi[r]) * p.H + qh[r]) * kDQ + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[r][ks] = *reinterpret_cast<const bf16x8*>(q + 32 * ks);
      m_ref[r] = -INFINITY;
      l_run[r] = 0.f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) acc[r][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    qk_scale = p.scale * kLog2e;
    {
      const int sw = swz(col);
      const int lo2 = (grp ^ sw) & 3;
      s_base_even = col * kRowBytes + 16 * ((0 ^ (sw & 4)) | lo2);
      s_base_odd = col * kRowBytes + 16 * ((4 ^ (sw & 4)) | lo2);
      const int src = 4 * grp + (col >> 2);    // token row fed by this lane (relative to t0)
      const int sw2 = swz(src);
      const int m4 = col & 3;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        v_base[q4] = src * kRowBytes + 16 * ((2 * q4 + (m4 >> 1)) ^ sw2) + 8 * (m4 & 1);
    }

    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // ids, queries and the first tile
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      if (i < nb) g_ids[i] = (idr[u] < 0 || idr[u] >= p.num_blocks) ? -1 : idr[u];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
    for (int i = 0; i < nb; ++i) bad |= g_ids[i] < 0;   // uniform: every lane reads all ids
    const int nb_run = bad ? 0 : nb;
    nb = nb_run;
    // Blocks alternate buffers 0 and 1 in pairs.
    if (nb > 0) {
      for (int k = 0; k < nb; k += 2) {
        step<0>(k);
        step<1>(k + 1);
      }
      wait_vmcnt<0>();
      lds_barrier();   // every wave's last copy has landed before LDS is reused below
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) l_run[r] = xor_sum(l_run[r]);
    if (TG == 2) {   // merge the two token halves of each row tile through LDS
      float* xo = reinterpret_cast<float*>(g_tile0);        // [WR][RPW][FT][64 lanes][4]
      float* xm = reinterpret_cast<float*>(g_tile1);        // [WR][RPW][64]
      float* xl = xm + WR * RPW * 64;
      if (tg == 1) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
#pragma unroll
          for (int ft = 0; ft < FT; ++ft)
            *reinterpret_cast<f32x4*>(xo + (((wr * RPW + r) * FT + ft) * 64 + lane) * 4) = acc[r][ft];
          xm[(wr * RPW + r) * 64 + lane] = m_ref[r];
          xl[(wr * RPW + r) * 64 + lane] = l_run[r];
        }
      }
      __syncthreads();
      if (tg == 1) return;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float m1 = xm[(wr * RPW + r) * 64 + lane], l1 = xl[(wr * RPW + r) * 64 + lane];
        const float M = fmaxf(m_ref[r], m1);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float w0 = __builtin_amdgcn_exp2f(m_ref[r] - M_use), w1 = __builtin_amdgcn_exp2f(m1 - M_use);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + (((wr * RPW + r) * FT + ft) * 64 + lane) * 4);
          acc[r][ft] = acc[r][ft] * w0 + o1 * w1;
        }
        l_run[r] = l_run[r] * w0 + l1 * w1;
        m_ref[r] = M;
      }
    }
    store();
  }

  __device__ __forceinline__ void store() {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t orow = static_cast<int64_t>(b * p.s_q + qi[r]) * p.H + qh[r];
      const bool empty = !(l_run[r] > 0.f);
      const float inv = empty ? 0.f : 1.f / l_run[r];
      float* dst = (p.n_split == 1 ? static_cast<float*>(p.out) + orow * kDC
                                   : p.ws_o + (orow * p.n_split + split) * kDC) + 4 * grp;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        f32x4 v = acc[r][ft] * inv;
        if (bad) v = f32x4{nan_f32(), nan_f32(), nan_f32(), nan_f32()};
        *reinterpret_cast<f32x4*>(dst + 16 * ft) = v;
      }
      if (grp == 0) {
        const float lse = bad ? nan_f32() : (empty ? -INFINITY : (m_ref[r] + __log2f(l_run[r])) * kLn2);
        if (p.n_split == 1) {
          if (p.lse != nullptr) p.lse[orow] = lse;
        } else {
          p.ws_lse[orow * p.n_split + split] = lse;
        }
      }
    }
  }
};

// P operands and rescale factors that the two waves of a feature-split pair swap each
// step: per wave, 2 halves x 64 lanes x 16 bytes, then 16 floats.
constexpr int kXchgWave = 2 * 1024 + 64;
__shared__ __attribute__((aligned(16))) char g_xchg[4 * kXchgWave];

// Feature-split variant: waves come in pairs over two 16-row tiles. Each wave scores its
// own tile (as above), the pair swaps the resulting P^T operands through LDS, and then
// each wave applies the value operands it reads to BOTH tiles for one half of the 512
// latent features. Every transposed LDS read (the most expensive LDS access here) thus
// feeds two MFMAs, halving that traffic, while the accumulator stays 2 x 256 x 16 rows.
// RT = row tiles per workgroup (2 or 4), TG = waves splitting each tile's 32-token halves.
template <int RT, int TG>
struct AbsorbPairCta {
  static constexpr int PR = RT / 2;                            // pairs
  static constexpr int W = RT * TG;                            // waves
  static constexpr int NH = 2 / TG;                            // 32-token halves per wave per tile
  static constexpr int PER_WAVE = kChunks * kBlock / 64 / W;   // 1 KiB copies per wave per tile
  static_assert(W == 4, "exchange area sized for 4 waves");
  static_assert(PER_WAVE * W * 64 == kChunks * kBlock, "tile must split evenly over waves");
  static_assert((PER_WAVE * 64) % (16 * kChunks) == 0, "wave copy block must hold whole swizzle periods");
  static_assert(PER_WAVE % NH == 0, "copies split over the halves");
  static constexpr int FH = kDC / 16 / 2;                      // feature tiles per half (16)
  static constexpr int KS = kDQ / 32;

  const AttnParams& p;
  int lane, wave, pair, fh, tg, col, grp;
  int b, split, part, L, blk_lo, nb;
  bool bad;
  int qi, qh, n_vis;
  bf16x8 qf[KS];
  f32x4 acc_own[FH], acc_par[FH];   // rows of this wave's tile / of the partner's tile
  float m_ref, l_run;               // this wave's tile
  float qk_scale;
  int s_base_even, s_base_odd;
  int v_base[4];
  uint32_t dma_off[PER_WAVE];

  __device__ AbsorbPairCta(const AttnParams& p_) : p(p_) {}

  __device__ __forceinline__ const char* tile_src(int k) const {
    const int32_t id = max(g_ids[k], 0);
    return static_cast<const char*>(p.kv) + static_cast<int64_t>(id) * kTileBytes + wave * PER_WAVE * 1024;
  }
  template <int BUF, int J>
  __device__ __forceinline__ void issue_one(const char* src) {
    copy16_to_lds(src + dma_off[J], (lds_void*)(tile_buf<BUF>() + (wave * PER_WAVE + J) * 1024));
  }
  template <int BUF, int J = 0>
  __device__ __forceinline__ void issue_all(const char* src) {
    if constexpr (J < PER_WAVE) {
      issue_one<BUF, J>(src);
      issue_all<BUF, J + 1>(src);
    }
  }
  template <int BUF, int J0, int J = J0>
  __device__ __forceinline__ void copy_at(int j, const char* src) {
    if constexpr (J < PER_WAVE) {
      if (j == J - J0) issue_one<BUF, J>(src);
      else copy_at<BUF, J0, J + 1>(j, src);
    }
  }

  template <int BUF>
  __device__ __forceinline__ void clear_tail(int valid) {
    char* tile = tile_buf<BUF>();
    for (int i = valid * kChunks + threadIdx.x; i < kBlock * kChunks; i += W * 64)
      *reinterpret_cast<uint4*>(tile + 16 * i) = uint4{0u, 0u, 0u, 0u};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
  }

  // Scores S^T = C Q^T of tokens t0 .. t0+31 for this wave's tile, with copies
  // J0 .. J0+CNT-1 of the next tile riding along (same scheme as AbsorbCta::score).
  template <int BUF, int J0, int CNT>
  __device__ __forceinline__ void score(int t0, f32x4 (&s)[2], const char* nxt) {
    const char* tile = tile_buf<BUF>() + t0 * kRowBytes;
    constexpr int N = 2 * KS;
    constexpr int D = kScoreBatch;
    static_assert(N % D == 0, "score batches");
    auto ld = [&](int i) {
      const int ks = i >> 1, tt = i & 1;
      return *reinterpret_cast<const bf16x8*>(tile + tt * 16 * kRowBytes + ((ks & 1) ? s_base_odd : s_base_even) +
                                              128 * (ks >> 1));
    };
    s[0] = s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a[N];
#pragma unroll
    for (int i = 0; i < D; ++i) a[i] = ld(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], qf[i >> 1], s[i & 1], 0, 0, 0);
      if (i % D == 0 && i + D < N) {
#pragma unroll
        for (int j = 0; j < D; ++j) a[i + D + j] = ld(i + D + j);
      }
      constexpr int GAP = N / CNT;
      if (i % GAP == GAP - 1 && i / GAP < CNT && nxt != nullptr) copy_at<1 - BUF, J0>(i / GAP, nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // O^T += C^T P^T over tokens t0 .. t0+31 for latent features fh*256 .. +256 and both
  // tiles of the pair: one transposed operand read per feature tile, two MFMAs.
  template <int BUF>
  __device__ __forceinline__ void value(int t0, bf16x8 p_own, bf16x8 p_par) {
    const char* tile = tile_buf<BUF>() + t0 * kRowBytes + fh * 512;   // 128 B per 4 feature tiles
    constexpr int D = kValueBatch;
    static_assert(FH % D == 0, "value batches");
    auto tr = [&](int ft, int second) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(tile + v_base[ft & 3] + 128 * (ft >> 2) + second * 16 * kRowBytes));
    };
    i16x4 lo[FH], hi[FH];
#pragma unroll
    for (int ft = 0; ft < D; ++ft) { lo[ft] = tr(ft, 0); hi[ft] = tr(ft, 1); }
#pragma unroll
    for (int ft = 0; ft < FH; ++ft) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[ft], hi[ft], 0, 1, 2, 3, 4, 5, 6, 7));
      acc_own[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, p_own, acc_own[ft], 0, 0, 0);
      acc_par[ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, p_par, acc_par[ft], 0, 0, 0);
      if (ft % D == 0 && ft + D < FH) {
#pragma unroll
        for (int j = 0; j < D; ++j) { lo[ft + D + j] = tr(ft + D + j, 0); hi[ft + D + j] = tr(ft + D + j, 1); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ char* xchg(int w) { return g_xchg + w * kXchgWave; }

  template <int BUF>
  __device__ __forceinline__ void step(int k) {
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (k < nb) {
      const int blk = blk_lo + k;
      const char* nxt = k + 1 < nb ? tile_src(k + 1) : nullptr;
      if ((blk + 1) * kBlock > L) clear_tail<BUF>(L - blk * kBlock);
      // Scores of this wave's halves (h0 = the first one).
      const int h0 = TG == 2 ? tg : 0;
      f32x4 s[NH][2];
      score<BUF, 0, PER_WAVE / NH>(h0 * 32, s[0], nxt);
      if constexpr (NH == 2) score<BUF, PER_WAVE / 2, PER_WAVE / 2>(32, s[1], nxt);
      // Online softmax over all of them: one max, lazy rescale (factor 1 when unchanged).
      float sc[NH][8];
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int tb = blk * kBlock + (h0 + h) * 32 + 4 * grp;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            const float v = (tb + 16 * tt + k2 < n_vis) ? s[h][tt][k2] * qk_scale : -INFINITY;
            sc[h][4 * tt + k2] = v;
            mx = fmaxf(mx, v);
          }
      }
      mx = xor_max(mx);
      float alpha = 1.f;
      if (mx > m_ref + kRescaleSlack) {
        alpha = __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
      }
      l_run *= alpha;
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      bf16x8 pf[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = __builtin_amdgcn_exp2f(sc[h][j] - m_use);
          l_run += e;
          pf[h][j] = static_cast<__bf16>(e);
        }
      // Swap P^T operands and rescale factors with the partner wave.
      char* mine = xchg(wave);
#pragma unroll
      for (int h = 0; h < NH; ++h) *reinterpret_cast<bf16x8*>(mine + h * 1024 + 16 * lane) = pf[h];
      if (grp == 0) reinterpret_cast<float*>(mine + 2048)[col] = alpha;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();
      const char* theirs = xchg(wave ^ 1);
      bf16x8 pp[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) pp[h] = *reinterpret_cast<const bf16x8*>(theirs + h * 1024 + 16 * lane);
      const float alpha_par = reinterpret_cast<const float*>(theirs + 2048)[col];
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f || alpha_par != 1.f) != 0) {   // rare after the first block
#pragma unroll
        for (int ft = 0; ft < FH; ++ft) {
          acc_own[ft] *= alpha;
          acc_par[ft] *= alpha_par;
        }
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) value<BUF>((h0 + h) * 32, pf[h], pp[h]);
    }
    // No closing barrier (see AbsorbCta::step); the exchange area is rewritten only after
    // the next opening barrier too.
  }

  __device__ __forceinline__ void run(int unit, int part_) {
    part = part_;
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    fh = wave & 1;
    pair = (wave >> 1) % PR;
    tg = (wave >> 1) / PR;
    col = lane & 15;
    grp = lane >> 4;
    split = unit % p.n_split;
    b = unit / p.n_split;
    L = p.ctx_lens[b];
    const int nblk = (L + kBlock - 1) / kBlock;
    bad = (L < p.s_q) || (L > p.max_blocks * kBlock) || (nblk > p.n_split * p.blocks_per_split);
    blk_lo = split * p.blocks_per_split;
    const int blk_hi = bad ? blk_lo : min(nblk, blk_lo + p.blocks_per_split);
    nb = max(0, blk_hi - blk_lo);
    // The first tile's copy starts before the rest of the prologue; the block ids (staged
    // in LDS, -1 marking an id outside the pool) and the queries load while it runs.
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dma_off[j] = slot_source(j * 64 + lane);
    const int32_t* table = p.block_table + static_cast<int64_t>(b) * p.max_blocks + blk_lo;
    if (nb > 0) {
      const int32_t id0 = table[0];
      const int32_t c0 = (id0 < 0 || id0 >= p.num_blocks) ? 0 : id0;   // a bad id poisons the output anyway
      issue_all<0>(static_cast<const char*>(p.kv) + static_cast<int64_t>(c0) * kTileBytes + wave * PER_WAVE * 1024);
    }
    constexpr int kIdsPerThread = kMaxSplitBlocks / (W * 64);
    int32_t idr[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      idr[u] = i < nb ? table[i] : 0;
    }
    // This wave scores tile 2*pair + fh: row = (part * RT + 2 * pair + fh) * 16 + col.
    {
      const int row = (part * RT + 2 * pair + fh) * 16 + col;
      qi = row / p.H;
      qh = row % p.H;
      n_vis = L - p.s_q + 1 + qi;
      const bf16_t* q = static_cast<const bf16_t*>(p.q) +
                        (static_cast<int64_t>(b * p.s_q + qi) * p.H + qh) * kDQ + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(q + 32 * ks);
    }
    m_ref = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int ft = 0; ft < FH; ++ft) acc_own[ft] = acc_par[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    qk_scale = p.scale * kLog2e;
    {
      const int sw = swz(col);
      const int lo2 = (grp ^ sw) & 3;
      s_base_even = col * kRowBytes + 16 * ((0 ^ (sw & 4)) | lo2);
      s_base_odd = col * kRowBytes + 16 * ((4 ^ (sw & 4)) | lo2);
      const int src = 4 * grp + (col >> 2);
      const int sw2 = swz(src);
      const int m4 = col & 3;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        v_base[q4] = src * kRowBytes + 16 * ((2 * q4 + (m4 >> 1)) ^ sw2) + 8 * (m4 & 1);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // ids, queries and the first tile
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      if (i < nb) g_ids[i] = (idr[u] < 0 || idr[u] >= p.num_blocks) ? -1 : idr[u];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
    for (int i = 0; i < nb; ++i) bad |= g_ids[i] < 0;
    nb = bad ? 0 : nb;
    if (nb > 0) {
      for (int k = 0; k < nb; k += 2) {
        step<0>(k);
        step<1>(k + 1);
      }
      wait_vmcnt<0>();
      lds_barrier();
    }

    // Row statistics of every tile and token group: ml[tg][tile][16] (m, then l).
    l_run = xor_sum(l_run);
    float* ml = reinterpret_cast<float*>(g_xchg);
    const int my_tile = 2 * pair + fh;
    if (grp == 0) {
      ml[((tg * RT + my_tile) * 2 + 0) * 16 + col] = m_ref;
      ml[((tg * RT + my_tile) * 2 + 1) * 16 + col] = l_run;
    }
    // Token group 1 hands its accumulators to token group 0 (tile buffers are free now).
    float* xo = reinterpret_cast<float*>(g_tile0);   // [pair][fh][own/par][FH][64 lanes][4]
    auto xo_at = [&](int j, int ft) { return xo + ((((pair * 2 + fh) * 2 + j) * FH + ft) * 64 + lane) * 4; };
    if (TG == 2 && tg == 1) {
#pragma unroll
      for (int ft = 0; ft < FH; ++ft) {
        *reinterpret_cast<f32x4*>(xo_at(0, ft)) = acc_own[ft];
        *reinterpret_cast<f32x4*>(xo_at(1, ft)) = acc_par[ft];
      }
    }
    __syncthreads();
    if (TG == 2 && tg == 1) return;
    store_tile(acc_own, my_tile, 0, ml, xo_at, true);
    store_tile(acc_par, 2 * pair + (fh ^ 1), 1, ml, xo_at, false);
  }

  // Merge (TG = 2) and store this wave's feature half of tile `tile` (rows of `acc`).
  template <typename XO>
  __device__ __forceinline__ void store_tile(f32x4 (&acc)[FH], int tile, int j, const float* ml, XO xo_at, bool lse_owner) {
    float m = ml[((0 * RT + tile) * 2 + 0) * 16 + col];
    float l = ml[((0 * RT + tile) * 2 + 1) * 16 + col];
    if constexpr (TG == 2) {
      const float m1 = ml[((1 * RT + tile) * 2 + 0) * 16 + col];
      const float l1 = ml[((1 * RT + tile) * 2 + 1) * 16 + col];
      const float M = fmaxf(m, m1);
      const float M_use = (M == -INFINITY) ? 0.f : M;
      const float w0 = __builtin_amdgcn_exp2f(m - M_use), w1 = __builtin_amdgcn_exp2f(m1 - M_use);
#pragma unroll
      for (int ft = 0; ft < FH; ++ft) acc[ft] = acc[ft] * w0 + *reinterpret_cast<const f32x4*>(xo_at(j, ft)) * w1;
      l = l * w0 + l1 * w1;
      m = M;
    }
    const int row = (part * RT + tile) * 16 + col;
    const int qi_t = row / p.H, qh_t = row % p.H;
    const int64_t orow = static_cast<int64_t>(b * p.s_q + qi_t) * p.H + qh_t;
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    float* dst = (p.n_split == 1 ? static_cast<float*>(p.out) + orow * kDC
                                 : p.ws_o + (orow * p.n_split + split) * kDC) + fh * 256 + 4 * grp;
#pragma unroll
    for (int ft = 0; ft < FH; ++ft) {
      f32x4 v = acc[ft] * inv;
      if (bad) v = f32x4{nan_f32(), nan_f32(), nan_f32(), nan_f32()};
      *reinterpret_cast<f32x4*>(dst + 16 * ft) = v;
    }
    if (lse_owner && grp == 0) {
      const float lse = bad ? nan_f32() : (empty ? -INFINITY : (m + __log2f(l)) * kLn2);
      if (p.n_split == 1) {
        if (p.lse != nullptr) p.lse[orow] = lse;
      } else {
        p.ws_lse[orow * p.n_split + split] = lse;
      }
    }
  }
};

// The H * s_q rows of a sequence are split into `parts` workgroups of RT * 16 rows. The
// parts of one (sequence, split) unit get workgroup ids 8 apart, which the dispatcher
// places on the same XCD, so each latent tile is read from HBM once and from that
// XCD's L2 by the other parts.
template <int RPW, int RT, int TG>
__global__ __launch_bounds__(RT / RPW * TG * 64, 1) void absorb_decode_split(AttnParams p, int parts, int units) {
  const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
  const int unit = parts == 1 ? static_cast<int>(blockIdx.x) : (y / parts) * 8 + x;
  const int part = parts == 1 ? 0 : y % parts;
  if (unit >= units) return;
  AbsorbCta<RPW, RT, TG> cta(p);
  cta.run(unit, part);
}

template <int RPW, int RT, int TG>
hipError_t launch(const AttnParams& p, int parts, hipStream_t s) {
  if (p.blocks_per_split > kMaxSplitBlocks) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(p.B) * p.n_split;
  const int64_t grid = parts == 1 ? units : ((units * parts + 8 * parts - 1) / (8 * parts)) * (8 * parts);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  absorb_decode_split<RPW, RT, TG><<<static_cast<unsigned>(grid), RT / RPW * TG * 64, 0, s>>>(p, parts, static_cast<int>(units));
  return hipGetLastError();
}

template <int RT, int TG>
__global__ __launch_bounds__(RT * TG * 64, 1) void absorb_decode_pair(AttnParams p, int parts, int units) {
  const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
  const int unit = parts == 1 ? static_cast<int>(blockIdx.x) : (y / parts) * 8 + x;
  const int part = parts == 1 ? 0 : y % parts;
  if (unit >= units) return;
  AbsorbPairCta<RT, TG> cta(p);
  cta.run(unit, part);
}

template <int RT, int TG>
hipError_t launch_pair(const AttnParams& p, int parts, hipStream_t s) {
  if (p.blocks_per_split > kMaxSplitBlocks) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(p.B) * p.n_split;
  const int64_t grid = parts == 1 ? units : ((units * parts + 8 * parts - 1) / (8 * parts)) * (8 * parts);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  absorb_decode_pair<RT, TG><<<static_cast<unsigned>(grid), RT * TG * 64, 0, s>>>(p, parts, static_cast<int>(units));
  return hipGetLastError();
}

int absorb_parts(const gqla_dims* d) {
  const int rows = d->num_heads * d->s_q;
  return rows > 64 ? rows / 64 : 1;
}

}  // namespace

bool tuned_absorb_supported(const gqla_dims* d) {
  const int rows = d->num_heads * d->s_q;
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->rope_dim == kDQ - kDC &&
         (rows == 16 || rows == 32 || rows == 64 || rows == 128 || rows == 256 || rows == 512);
}

// One 156 KiB workgroup per CU; each (sequence, split) unit takes absorb_parts() of them.
int tuned_absorb_target_wgs(const gqla_dims* d) { return kNumCUs / absorb_parts(d); }

int tuned_absorb_min_blocks_per_split() { return 4; }

int tuned_absorb_max_blocks_per_split() { return kMaxSplitBlocks; }

hipError_t launch_tuned_absorb(const AttnParams& p, const gqla_dims* d, hipStream_t s) {
  switch (d->num_heads * d->s_q) {
    // At 32 rows the pair's extra exchange barrier costs more than the halved transposed
    // reads save (measured 74 vs 71 us on LLaMA-3-8B batch 32); from 64 rows on the pair wins.
    case 16: return launch<1, 1, 2>(p, 1, s);
    case 32: return launch<1, 2, 2>(p, 1, s);
    case 64: return launch_pair<4, 1>(p, 1, s);
    case 128: return launch_pair<4, 1>(p, 2, s);
    case 256: return launch_pair<4, 1>(p, 4, s);
    case 512: return launch_pair<4, 1>(p, 8, s);
  }
  return hipErrorNotSupported;
}

}  // namespace gqla
