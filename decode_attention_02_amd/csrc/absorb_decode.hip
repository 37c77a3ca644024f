// MQA-absorb split-KV decode on gfx950 MFMA (bf16 latent, fp32 accumulation).
//
// Every query head, with W_UK^g folded into it, attends over the one shared latent
// "key head" [c_KV | k_rope] and takes the latent c_KV itself as its value (MLA's
// absorbed form, which GQLA keeps unchanged: "GQLA: Attention latente ...", English
// abstract; gqla_attn.py docstring: a single MQA-style head per layer).
//
// All H * s_q query rows of a sequence read the same latent tiles, so a tile is fetched
// from HBM once per workgroup and shared through LDS:
//   * tiles (64 tokens x 576 bf16 = 72 KiB, or 32-token sub-tiles) are copied
//     global -> LDS by global_load_lds_dwordx4 (no register staging), with an XOR
//     swizzle of the 16-byte chunks inside each 128-byte group so that both LDS
//     access patterns below are bank-conflict free;
//   * scores S^T = C Q^T (v_mfma_f32_16x16x32_bf16, A = 16 tokens x 32 latent features
//     read with ds_read_b128, B = absorbed queries held in registers);
//   * the value product O^T = C^T P^T needs the latent with tokens along the
//     contraction, which ds_read_b64_tr_b16 delivers directly from the row-major tile;
//     P is the B operand;
//   * 16 or 32 rows (AbsorbCta, bound by HBM): each wave owns 16 query rows for both
//     products and each double-buffered tile's two 32-token halves go to two waves,
//     merged at the end, so a workgroup still has 4 waves streaming;
//   * 64 rows and more (AbsorbSpecCta, bound by the matrix cores): 64 rows per
//     workgroup of eight waves, four forming scores and P (two row tiles and one
//     16-token half each, so each operand read feeds two MFMAs) and four applying P to a
//     quarter of the latent features of all rows (each transposed read feeding four
//     MFMAs), one 32-token sub-tile apart, with P exchanged through LDS; 128 to 512 rows
//     use 2 to 8 such workgroups per (sequence, split), placed on the same XCD so the
//     repeated tile reads are served from that XCD's L2.
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

// Swizzle of a token row's 16-byte chunk index inside its 128-byte group (chunk c of row t
// is stored at c xor swz(t)): the score operand reads take one chunk of each of 16 rows,
// the transposed reads a chunk pair of each of 16 rows. swz(t) = 2 (t0 xor t3) + 4 t1 (bits
// of t) keeps each chunk pair together and has period 16, so every read base that is a
// multiple of 16 rows sees the same pattern. Chosen by measurement: against
// (t mod 8) xor t3 it halves the LDS bank-conflict cycles of the specialized-wave decode
// (SQ_LDS_BANK_CONFLICT 34% -> 20% of SQ_LDS_IDX_ACTIVE) with bit-identical results.
__device__ __forceinline__ int swz(int t) { return 2 * ((t ^ (t >> 3)) & 1) + 4 * ((t >> 1) & 1); }

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48) with
// gfx950's row-swap instructions: v_permlane16_swap exchanges rows 0 <-> 1 and 2 <-> 3
// between its two operands, v_permlane32_swap the two 32-lane halves, so with both
// operands holding v each lane ends up with its own value in one result and its
// partner's in the other. Plain VALU operations, unlike the LDS round trip of a shuffle.
__device__ __forceinline__ float xor_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float xor_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
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
__shared__ int32_t g_touch[64];          // landing place of the translation touches (never read)

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


  // One dword of the wave's part of block k, loaded by one lane two steps before its copy:
  // with a shuffled block table over a large pool most blocks sit on pages whose address
  // translation is not cached, and the touch starts that translation early (0.6-1.1% faster
  // on the one-eighth DeepSeek-V3 share at batch 10240 x 16K, 180 GiB of latent, at s_q = 1
  // and 2; no change at 36 GiB). Every step opens by waiting for all of the wave's loads, so
  // the touch needs no count of its own.
  __device__ __forceinline__ void touch(int k) {
    if (k < nb && lane == 0)
      __builtin_amdgcn_global_load_lds(tile_src(k), (lds_void*)(g_touch + wave), 4, 0, 0);
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
  // since tok = t0 + 16*tt + col with t0 + 16*tt a multiple of 16, swz(tok) = swz(col)
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
      constexpr int GAP = CNT > 0 ? N / CNT : 1;
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
  // piecemeal from inside the score loop (all at once first in the 32-row form). The other buffer is free: every wave has passed
  // this step's opening barrier, so all of them are done reading it.
  template <int BUF>
  __device__ __forceinline__ void step(int k) {
    __builtin_amdgcn_s_waitcnt(0);   // this block's copy has landed, this wave's LDS reads are done
    lds_barrier();
    if (k < nb) {
      const int blk = blk_lo + k;
      const char* nxt = k + 1 < nb ? tile_src(k + 1) : nullptr;
      if ((blk + 1) * kBlock > L) clear_tail<BUF>(L - blk * kBlock);
      if constexpr (TG == 2 && RT == 2 && RPW == 1) {
        // 32 rows (HBM-bound): the next tile's copies all go out first, for the longest lead
        // (0.5-1% faster than spreading them over the score loop).
        if (nxt != nullptr) issue_all<1 - BUF>(nxt);
        touch(k + 2);
        half_step<BUF, 0, 0>(tg, blk, nxt);
      } else if constexpr (TG == 2) {
        touch(k + 2);
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

// ---------------------------------------------------------------------------------------
// 64 rows per workgroup with the two products on different waves: eight waves, two per
// SIMD, waves 0-3 forming scores and P, waves 4-7 applying P to the latent. The latent
// streams in 32-token sub-tiles through a ring of four LDS slots; iteration i:
//   * score wave (sg, th) forms S^T for rows 32 sg .. +32 (two row tiles, each operand read
//     feeding two MFMAs) over tokens 16 th .. +16 of sub-tile i, its online softmax against
//     its own running reference, and publishes P^T and that reference through LDS;
//   * value wave v copies sub-tile i + 2 into the free slot, zeroes the rows of sub-tile i
//     past the context, and applies P of sub-tile i - 1 to latent features 128 v .. +128 of
//     all four row tiles (each transposed read feeding four MFMAs), first raising its own
//     reference to the larger published one and rescaling what was formed against less.
// One barrier per iteration. The two waves of a SIMD have different roles, so one's
// exponentials and LDS waits run under the other's matrix work; each role keeps only its
// own state (queries or accumulators) within 256 registers.
constexpr int kSubTok = 32;
constexpr int kSubBytes = kSubTok * kRowBytes;    // 36864
constexpr int kSubCopies = kSubBytes / 1024;      // 1 KiB copies per sub-tile (36)
__shared__ __attribute__((aligned(16))) char g_sub0[kSubBytes];
__shared__ __attribute__((aligned(16))) char g_sub1[kSubBytes];
__shared__ __attribute__((aligned(16))) char g_sub2[kSubBytes];
__shared__ __attribute__((aligned(16))) char g_sub3[kSubBytes];
__shared__ __attribute__((aligned(16))) char g_sp[2][4 * 64 * 16];   // P^T operands [buf][row tile][lane]
__shared__ float g_sm[2][4][2][16];   // reference of each published P [buf][row tile][th][row]
__shared__ float g_sl[4][2][16];      // final row sums of the score waves [row tile][th][row]
__shared__ float g_sr[4][2][16];      // and their final references

template <int S>
__device__ __forceinline__ char* sub_buf() {
  return S == 0 ? g_sub0 : S == 1 ? g_sub1 : S == 2 ? g_sub2 : g_sub3;
}

struct AbsorbSpecCta {
  static constexpr int W = 8;
  static constexpr int NT = 4;                  // row tiles
  static constexpr int KS = kDQ / 32;           // k-steps of the score product (18)
  static constexpr int FQ = kDC / 16 / 4;       // feature tiles per value wave (8)
  static constexpr int CPW = kSubCopies / 4;    // copies per value wave per sub-tile (9)
  static constexpr int SB = 9;                  // score operand reads per batch
  static constexpr int VB = 4;                  // value feature tiles per batch
  static constexpr int NA = 5;                  // copies a value wave issues after the barrier (the rest after its products)
  static_assert(KS % SB == 0 && FQ % VB == 0, "batches");
  static_assert(CPW * 4 == kSubCopies, "sub-tile copies split over the value waves");

  const AttnParams& p;
  int lane, wave, col, grp;
  int b, split, part, L, blk_lo, nb, n_sub;
  bool bad;

  __device__ AbsorbSpecCta(const AttnParams& p_) : p(p_) {}

  // Block ids of the split into LDS (-1 marks an id outside the pool), then the workgroup
  // agrees on `bad` and the number of blocks. Every wave runs this once.
  __device__ __forceinline__ void stage_ids() {
    const int32_t* table = p.block_table + static_cast<int64_t>(b) * p.max_blocks + blk_lo;
    constexpr int kIdsPerThread = kMaxSplitBlocks / (W * 64);
    int32_t idr[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      idr[u] = i < nb ? table[i] : 0;
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // ids, queries, the first copies
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
      const int i = threadIdx.x + u * W * 64;
      if (i < nb) g_ids[i] = (idr[u] < 0 || idr[u] >= p.num_blocks) ? -1 : idr[u];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
    for (int i = 0; i < nb; ++i) bad |= g_ids[i] < 0;
    nb = bad ? 0 : nb;
    n_sub = 2 * nb;
  }

  // ---- score waves ----
  struct Score {
    int sg, th;
    int n_vis[2];
    bf16x8 qf[2][KS];
    float m_ref[2], l_part[2];
    int s_base_even, s_base_odd;
  };

  template <int SLOT>
  __device__ __forceinline__ void score_step(Score& st, int i, float qk_scale) {
    const char* tile = sub_buf<SLOT>() + st.th * 16 * kRowBytes;
    auto ld = [&](int ks) {
      return *reinterpret_cast<const bf16x8*>(tile + ((ks & 1) ? st.s_base_odd : st.s_base_even) + 128 * (ks >> 1));
    };
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    bf16x8 a[KS];
#pragma unroll
    for (int k = 0; k < SB; ++k) a[k] = ld(k);
    // The other token half's references of the previous sub-tile, read under the MFMAs.
    float other[2] = {-INFINITY, -INFINITY};
    if (i > 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) other[j] = g_sm[(i - 1) & 1][2 * st.sg + j][1 - st.th][col];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < 2; ++j) s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], st.qf[j][ks], s[j], 0, 0, 0);
      if (ks % SB == 0 && ks + SB < KS) {
#pragma unroll
        for (int k = 0; k < SB; ++k) a[ks + SB + k] = ld(ks + SB + k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Lane (row col, grp) holds tokens 16 th + 4 grp + r of the sub-tile, r = 0..3.
    const int tb = blk_lo * kBlock + i * kSubTok + 16 * st.th + 4 * grp;
    char* pbuf = g_sp[i & 1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 2 * st.sg + j;
      // Adopt the other token half's reference from the previous sub-tile when larger, so
      // that both halves publish P against the same reference and the value waves rarely
      // have to rescale it.
      if (other[j] > st.m_ref[j]) {
        if (st.m_ref[j] != -INFINITY) st.l_part[j] *= __builtin_amdgcn_exp2f(st.m_ref[j] - other[j]);
        st.m_ref[j] = other[j];
      }
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = (tb + r < st.n_vis[j]) ? s[j][r] * qk_scale : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      mx = xor_max(mx);
      if (mx > st.m_ref[j] + kRescaleSlack) {
        if (st.m_ref[j] != -INFINITY) st.l_part[j] *= __builtin_amdgcn_exp2f(st.m_ref[j] - mx);
        st.m_ref[j] = mx;
      }
      const float m_use = (st.m_ref[j] == -INFINITY) ? 0.f : st.m_ref[j];
      __bf16 pv[4];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(sc[r] - m_use);
        ls += e;
        pv[r] = static_cast<__bf16>(e);
      }
      st.l_part[j] += ls;
      *reinterpret_cast<uint2*>(pbuf + (t * 64 + lane) * 16 + st.th * 8) = __builtin_bit_cast(uint2, pv);
      if (grp == 0) g_sm[i & 1][t][st.th][col] = st.m_ref[j];
    }
  }

  // One iteration of the score waves; false once past the last one.
  template <int U>
  __device__ __forceinline__ bool score_iter(Score& st, int i, float qk_scale) {
    if (i > n_sub) return false;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's P and references are written
    lds_barrier();
    if (i < n_sub) score_step<U>(st, i, qk_scale);
    return true;
  }

  __device__ void run_score() {
    Score st;
    st.sg = wave >> 1;
    st.th = wave & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = (part * NT + 2 * st.sg + j) * 16 + col;
      const int qi = row / p.H, qh = row % p.H;
      st.n_vis[j] = L - p.s_q + 1 + qi;
      const bf16_t* q = static_cast<const bf16_t*>(p.q) +
                        (static_cast<int64_t>(b * p.s_q + qi) * p.H + qh) * kDQ + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st.qf[j][ks] = *reinterpret_cast<const bf16x8*>(q + 32 * ks);
      st.m_ref[j] = -INFINITY;
      st.l_part[j] = 0.f;
    }
    {
      const int sw = swz(col);
      const int lo2 = (grp ^ sw) & 3;
      st.s_base_even = col * kRowBytes + 16 * ((0 ^ (sw & 4)) | lo2);
      st.s_base_odd = col * kRowBytes + 16 * ((4 ^ (sw & 4)) | lo2);
    }
    const float qk_scale = p.scale * kLog2e;
    stage_ids();
    if (nb > 0) {
      for (int i = 0;; i += 4) {
        if (!score_iter<0>(st, i, qk_scale) || !score_iter<1>(st, i + 1, qk_scale) ||
            !score_iter<2>(st, i + 2, qk_scale) || !score_iter<3>(st, i + 3, qk_scale))
          break;
      }
    }
    // Row sums (over the four lane groups) and final references for the value waves.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float l = xor_sum(st.l_part[j]);
      if (grp == 0) {
        g_sl[2 * st.sg + j][st.th][col] = l;
        g_sr[2 * st.sg + j][st.th][col] = st.m_ref[j];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
  }

  // ---- value waves ----
  struct Value {
    int v;
    f32x4 acc[NT][FQ];
    float mv[NT];          // reference of acc for row `col` of each tile (log2 domain)
    uint32_t coff[CPW];    // per-lane source offsets of this wave's copies within a sub-tile
    int v_base[4];
    i16x4 plo[VB], phi[VB];   // first batch of transposed reads of the next value step
  };

  // Copies of sub-tile k (block k / 2, half k % 2) into slot S. Cache-retaining loads: the
  // other row parts of the sequence (on the same XCD) read the same sub-tile from L2; with
  // non-temporal loads they missed there and HBM reads were 1.35-1.47x the latent bytes at
  // 128 and 256 rows, with these 1.03x.
  template <int S, int J0, int J1>
  __device__ __forceinline__ void issue_part(const Value& vt, const char* block) {
#pragma unroll
    for (int J = J0; J < J1; ++J)
      __builtin_amdgcn_global_load_lds(block + vt.coff[J], (lds_void*)(sub_buf<S>() + (vt.v * CPW + J) * 1024), 16, 0, 0);
  }
  template <int S>
  __device__ __forceinline__ void issue_sub(const Value& vt, const char* block) {
#pragma unroll
    for (int J = 0; J < CPW; ++J)
      __builtin_amdgcn_global_load_lds(block + vt.coff[J], (lds_void*)(sub_buf<S>() + (vt.v * CPW + J) * 1024), 16, 0, 0);
  }
  __device__ __forceinline__ const char* sub_src(int32_t id, int k) const {
    id = __builtin_amdgcn_readfirstlane(max(id, 0));
    return static_cast<const char*>(p.kv) + static_cast<int64_t>(id) * kTileBytes + (k & 1) * kSubBytes;
  }

  template <int SV>
  __device__ __forceinline__ i16x4 vtr(const Value& vt, int ft, int second) {
    const char* tile = sub_buf<SV>() + vt.v * 256;   // features 128 v .. +128
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + vt.v_base[ft & 3] + 128 * (ft >> 2) + second * 16 * kRowBytes));
  }
  // The first batch of the next value step's transposed reads, issued at the end of an
  // iteration: they land while the wave waits for the barrier.
  template <int SV>
  __device__ __forceinline__ void value_prefetch(Value& vt) {
#pragma unroll
    for (int ft = 0; ft < VB; ++ft) { vt.plo[ft] = vtr<SV>(vt, ft, 0); vt.phi[ft] = vtr<SV>(vt, ft, 1); }
  }
  __device__ __forceinline__ void read_mp(int k, float (&mh)[2][NT], bf16x8 (&pb)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) mh[h][t] = g_sm[k & 1][t][h][col];
    const char* pbuf = g_sp[k & 1];
#pragma unroll
    for (int t = 0; t < NT; ++t) pb[t] = *reinterpret_cast<const bf16x8*>(pbuf + (t * 64 + lane) * 16);
  }

  template <int SV>
  __device__ __forceinline__ void value_step(Value& vt, int k, float (&mh)[2][NT], bf16x8 (&pb)[NT]) {
    auto tr = [&](int ft, int second) { return vtr<SV>(vt, ft, second); };
    i16x4 lo[FQ], hi[FQ];
#pragma unroll
    for (int ft = 0; ft < VB; ++ft) { lo[ft] = vt.plo[ft]; hi[ft] = vt.phi[ft]; }
    bool mixed = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float M = fmaxf(mh[0][t], mh[1][t]);
      const bool grow = M > vt.mv[t];
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // rare after the first sub-tiles
        const float alpha = grow ? __builtin_amdgcn_exp2f(vt.mv[t] - M) : 1.f;   // 0 from -inf: acc is 0 then
#pragma unroll
        for (int ft = 0; ft < FQ; ++ft) vt.acc[t][ft] *= alpha;
        if (grow) vt.mv[t] = M;
      }
      mixed |= mh[0][t] != vt.mv[t] || mh[1][t] != vt.mv[t];
    }
    if (__builtin_amdgcn_ballot_w64(mixed) != 0) {   // a half formed against a smaller reference
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float f = mh[h][t] < vt.mv[t] ? __builtin_amdgcn_exp2f(mh[h][t] - vt.mv[t]) : 1.f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[t][4 * h + e] = static_cast<__bf16>(static_cast<float>(pb[t][4 * h + e]) * f);
        }
      }
    }
#pragma unroll
    for (int ft = 0; ft < FQ; ++ft) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[ft], hi[ft], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < NT; ++t) vt.acc[t][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[t], vt.acc[t][ft], 0, 0, 0);
      if (ft % VB == 0 && ft + VB < FQ) {
#pragma unroll
        for (int jj = 0; jj < VB; ++jj) { lo[ft + VB + jj] = tr(ft + VB + jj, 0); hi[ft + VB + jj] = tr(ft + VB + jj, 1); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Iteration i of the value waves (slot U = i % 4 holds sub-tile i, (U + 3) % 4 sub-tile
  // i - 1, (U + 2) % 4 receives sub-tile i + 2); false once past the last one.
  template <int U>
  __device__ __forceinline__ bool value_iter(Value& vt, int i) {
    if (i > n_sub) return false;
    // The copies always run: past the last sub-tile they repeat it into the free slot,
    // which keeps the count of copies in flight exact. Their block id is read from LDS
    // before the waits, which cover its latency.
    const int k_next = min(i + 2, n_sub - 1);
    const int32_t id_next = g_ids[k_next >> 1];
    wait_vmcnt<CPW>();                                   // sub-tile i has landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's zeroing and reads are done
    lds_barrier();
    // The copies of sub-tile i + 2 go out in two parts: NA right after the barrier, the rest
    // after this iteration's products, so the wait for room in the memory pipeline is split
    // between the two ends of the iteration (2% faster than all nine at the start).
    const char* csrc = sub_src(id_next, k_next);
    issue_part<(U + 2) % 4, 0, NA>(vt, csrc);
    // The references and P^T of sub-tile i - 1; the first half of its transposed latent reads
    // were issued at the end of the previous iteration, the second half goes out under the
    // first products.
    float mh[2][NT];
    bf16x8 pb[NT];
    if (i >= 1) read_mp(i - 1, mh, pb);
    if (i < n_sub) {   // rows of sub-tile i past the context: zero, so the value product needs no mask
      const int tok0 = (blk_lo * 2 + i) * kSubTok;
      if (tok0 + kSubTok > L) {
        // Each value wave zeroes the 16 chunks of its own features (the swizzle moves chunks
        // only within 8-chunk groups), so its own later reads need no barrier.
        char* tile = sub_buf<U>();
        const int valid = max(0, L - tok0);
        for (int q = lane; q < (kSubTok - valid) * 16; q += 64)
          *reinterpret_cast<uint4*>(tile + (valid + (q >> 4)) * kRowBytes + 16 * (16 * vt.v + (q & 15))) =
              uint4{0u, 0u, 0u, 0u};
      }
    }
    if (i >= 1) value_step<(U + 3) % 4>(vt, i - 1, mh, pb);
    issue_part<(U + 2) % 4, NA, CPW>(vt, csrc);
    if (i < n_sub) value_prefetch<U>(vt);
    return true;
  }

  __device__ void run_value() {
    Value vt;
    vt.v = wave - 4;
#pragma unroll
    for (int J = 0; J < CPW; ++J) vt.coff[J] = slot_source((vt.v * CPW + J) * 64 + lane);
    // The first two sub-tiles (block 0 of the split) are copied before the block ids are
    // staged; an id outside the pool is replaced by block 0 (it poisons the output anyway).
    if (nb > 0) {
      const int32_t id0 = p.block_table[static_cast<int64_t>(b) * p.max_blocks + blk_lo];
      const char* blk0 = static_cast<const char*>(p.kv) +
                         static_cast<int64_t>((id0 < 0 || id0 >= p.num_blocks) ? 0 : id0) * kTileBytes;
      issue_sub<0>(vt, blk0);
      issue_sub<1>(vt, blk0 + kSubBytes);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      vt.mv[t] = -INFINITY;
#pragma unroll
      for (int ft = 0; ft < FQ; ++ft) vt.acc[t][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    {
      const int src = 4 * grp + (col >> 2);
      const int sw2 = swz(src);
      const int m4 = col & 3;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vt.v_base[q4] = src * kRowBytes + 16 * ((2 * q4 + (m4 >> 1)) ^ sw2) + 8 * (m4 & 1);
    }
    stage_ids();
    if (nb > 0) {
      for (int i = 0;; i += 4) {
        if (!value_iter<0>(vt, i) || !value_iter<1>(vt, i + 1) || !value_iter<2>(vt, i + 2) ||
            !value_iter<3>(vt, i + 3))
          break;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the repeated copies have landed before the workgroup ends
    lds_barrier();                   // the score waves' row sums and references are written
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float l0 = g_sl[t][0][col], l1 = g_sl[t][1][col];
      const float r0 = g_sr[t][0][col], r1 = g_sr[t][1][col];
      const float M = vt.mv[t];
      const float M_use = (M == -INFINITY) ? 0.f : M;
      const float l = l0 * __builtin_amdgcn_exp2f(r0 - M_use) + l1 * __builtin_amdgcn_exp2f(r1 - M_use);
      const int row = (part * NT + t) * 16 + col;
      const int qi = row / p.H, qh = row % p.H;
      const int64_t orow = static_cast<int64_t>(b * p.s_q + qi) * p.H + qh;
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : 1.f / l;
      float* dst = (p.n_split == 1 ? static_cast<float*>(p.out) + orow * kDC
                                   : p.ws_o + (orow * p.n_split + split) * kDC) + vt.v * 128 + 4 * grp;
#pragma unroll
      for (int ft = 0; ft < FQ; ++ft) {
        f32x4 o = vt.acc[t][ft] * inv;
        if (bad) o = f32x4{nan_f32(), nan_f32(), nan_f32(), nan_f32()};
        *reinterpret_cast<f32x4*>(dst + 16 * ft) = o;
      }
      if (vt.v == 0 && grp == 0) {
        const float lse = bad ? nan_f32() : (empty ? -INFINITY : (M + __log2f(l)) * kLn2);
        if (p.n_split == 1) {
          if (p.lse != nullptr) p.lse[orow] = lse;
        } else {
          p.ws_lse[orow * p.n_split + split] = lse;
        }
      }
    }
  }

  __device__ __forceinline__ void run(int unit, int part_) {
    part = part_;
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    if (wave < 4) run_score();
    else run_value();
  }
};

__global__ __launch_bounds__(512, 1) void absorb_decode_spec(AttnParams p, int parts, int units) {
  const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
  const int unit = parts == 1 ? static_cast<int>(blockIdx.x) : (y / parts) * 8 + x;
  const int part = parts == 1 ? 0 : y % parts;
  if (unit >= units) return;
  AbsorbSpecCta cta(p);
  cta.run(unit, part);
}

hipError_t launch_spec(const AttnParams& p, int parts, hipStream_t s) {
  if (p.blocks_per_split > kMaxSplitBlocks) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(p.B) * p.n_split;
  const int64_t grid = parts == 1 ? units : ((units * parts + 8 * parts - 1) / (8 * parts)) * (8 * parts);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  absorb_decode_spec<<<static_cast<unsigned>(grid), 512, 0, s>>>(p, parts, static_cast<int>(units));
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

// One workgroup per CU (148-158 KiB of LDS); each (sequence, split) unit takes absorb_parts() of them.
int tuned_absorb_target_wgs(const gqla_dims* d) { return kNumCUs / absorb_parts(d); }

int tuned_absorb_min_blocks_per_split() { return 4; }

int tuned_absorb_max_blocks_per_split() { return kMaxSplitBlocks; }

hipError_t launch_tuned_absorb(const AttnParams& p, const gqla_dims* d, hipStream_t s) {
  switch (d->num_heads * d->s_q) {
    // Up to 32 rows each wave keeps its rows to itself: no P exchange, one barrier per
    // tile less (an exchanging layout measured 74 against 71 us on LLaMA-3-8B batch 32).
    // From 64 rows the products go to separate waves (AbsorbSpecCta).
    case 16: return launch<1, 1, 2>(p, 1, s);
    case 32: return launch<1, 2, 2>(p, 1, s);
    case 64: return launch_spec(p, 1, s);
    case 128: return launch_spec(p, 2, s);
    case 256: return launch_spec(p, 4, s);
    case 512: return launch_spec(p, 8, s);
  }
  return hipErrorNotSupported;
}

}  // namespace gqla
