// Output side of the attention layer on gfx950: the projection W_O that follows the heads
// (the module's bias-free out_proj over the head-major concatenation of the heads'
// outputs, "gqla_attn.py" module source, GQLAAttention.forward), and, for the MQA-absorb
// path, W_O with each head's value up-projection W_UV^g folded in.
//
//   unfolded:  y[r][n] = sum_{h,v} W_O[n][h*d_v + v]    out[r][h][v]     (out: bf16)
//   folded:    y[r][n] = sum_{h,c} W_fold[n][h*d_c + c] o_lat[r][h][c]   (o_lat: fp32)
//   fold:      W_fold[n][h*d_c + c] = sum_v W_O[n][h*d_v + v] W_UV^g[v][c]   (once per model)
//
// At decode there are few rows (B * s_q) against a large weight (hidden x H*d_v or
// hidden x H*d_c), so the product is bound by streaming the weight from HBM once. Each
// workgroup owns 16, 32 or 64 output features (rows of the weight) and splits the
// contraction over its 4 waves; every wave streams its part of those rows with 16-byte
// loads (the MFMA A operand straight from global memory, two chunks in flight) and reads
// the rows' inputs, which every workgroup shares, from L2, each input operand feeding
// one MFMA per weight tile. The 4 partial results are summed through LDS. An fp32 input
// is split into bf16 high and low parts (two MFMAs), which keeps the product close to fp32
// accuracy. With bf16 inputs, most shapes use a form that streams the weight through LDS in
// 512-byte runs per row (hidden_ks below); wide layers whose contraction is not whole
// 256-element chunks stage both operands through LDS in 256-byte runs (hidden_dma).
#include "device_common.h"
#include "gqla_internal.h"

#include <type_traits>

namespace gqla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // waves per workgroup, each a quarter of the contraction
constexpr int kU = 4;            // k-steps (of 32) per load chunk (2 for fp32 inputs)

// Weight rows n0 .. n0 + 16*NTW, input rows m0 .. m0 + 16*MT. Each input operand feeds
// NTW MFMAs and each weight operand MT (the weight is the HBM stream; the inputs, read by
// every workgroup, come from L2, so NTW >= MT keeps their traffic at or below the
// weight's).
template <bool XF32, int MT, int NTW>
__global__ __launch_bounds__(kWaves * 64) void hidden_gemm(const void* x, const bf16_t* w, bf16_t* y, int M, int N,
                                                            int K) {
  __shared__ f32x4 part[kWaves][NTW][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16 * NTW;
  const int m0 = blockIdx.y * 16 * MT;
  const int kw = K / kWaves;                    // a multiple of 32 (K % 128 == 0)
  const int kbeg = wave * kw;
  const int steps = kw / 32;
  // A operand of weight tile j: row n0 + 16*j + col, features k + 8*grp .. +8.
  const bf16_t* wrow = w + static_cast<int64_t>(n0 + col) * K + kbeg + 8 * grp;
  const int64_t wtile = static_cast<int64_t>(16) * K;
  // B operand: input row m (clamped to the last row; only live rows are stored).
  int64_t xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = static_cast<int64_t>(min(m0 + 16 * t + col, M - 1)) * K + kbeg + 8 * grp;

  f32x4 acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk = U k-steps of the weight tiles and of the input rows, loaded together.
  // Two chunks must fit in registers beside the accumulators: a chunk holding more than
  // 16 loads per lane would be parked in AGPRs, which waits for its loads at once.
  constexpr int U = (XF32 || NTW * MT > 4) ? 2 : kU;
  constexpr int XV = XF32 ? 2 : 1;               // 16-byte loads per input operand
  struct Chunk {
    bf16x8 w[U][NTW];
    f32x4 x[U][MT][XV];                         // bf16 inputs use the bits of x[..][0]
  };
  // Unconditional loads of chunk s0 .. s0 + U - 1 (always a whole chunk inside the range):
  // no branch around a load, so every load of a chunk is in flight at once.
  auto load = [&](Chunk& c, int s0, auto n) {
    constexpr int NU = decltype(n)::value;   // k-steps to load (U, or 1 for the tail)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) c.w[u][j] = *reinterpret_cast<const bf16x8*>(wrow + j * wtile + 32 * (s0 + u));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if constexpr (XF32) {
          const float* xp = static_cast<const float*>(x) + xrow[t] + 32 * (s0 + u);
          c.x[u][t][0] = *reinterpret_cast<const f32x4*>(xp);
          c.x[u][t][1] = *reinterpret_cast<const f32x4*>(xp + 4);
        } else {
          c.x[u][t][0] = *reinterpret_cast<const f32x4*>(static_cast<const bf16_t*>(x) + xrow[t] + 32 * (s0 + u));
        }
      }
    }
  };
  auto mma = [&](const Chunk& c, auto n) {
    constexpr int NU = decltype(n)::value;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if constexpr (XF32) {
          bf16x8 hi, lo;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float v = c.x[u][t][k >> 2][k & 3];
            const __bf16 h = static_cast<__bf16>(v);
            hi[k] = h;
            lo[k] = static_cast<__bf16>(v - static_cast<float>(h));
          }
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.w[u][j], hi, acc[j][t], 0, 0, 0);
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.w[u][j], lo, acc[j][t], 0, 0, 0);
          }
        } else {
          const bf16x8 xv = __builtin_bit_cast(bf16x8, c.x[u][t][0]);
#pragma unroll
          for (int j = 0; j < NTW; ++j) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.w[u][j], xv, acc[j][t], 0, 0, 0);
        }
      }
    }
  };

  // Two chunks in flight: the next chunk's loads go out before this one is used. Whole
  // chunks first (past the last one the last is loaded again, an L2 hit left unused), then
  // the k-steps that do not fill a chunk one at a time.
  const int nch = steps / U;
  int ch = 0;
  if (nch > 0) {
    const std::integral_constant<int, U> whole;
    Chunk ca, cb;
    load(ca, 0, whole);
    for (; ch + 1 < nch; ch += 2) {
      load(cb, (ch + 1) * U, whole);
      __builtin_amdgcn_sched_barrier(0);
      mma(ca, whole);
      load(ca, min(ch + 2, nch - 1) * U, whole);
      __builtin_amdgcn_sched_barrier(0);
      mma(cb, whole);
    }
    if (ch < nch) mma(ca, whole);
  }
  for (int s1 = nch * U; s1 < steps; ++s1) {
    const std::integral_constant<int, 1> one;
    Chunk c1;
    load(c1, s1, one);
    mma(c1, one);
  }

  // D[n][m]: lane holds features n0 + 16*j + 4*grp + r of row m0 + 16*t + col. Sum the
  // waves' shares; wave j' stores weight tiles j = j', j' + 4, ...
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) part[wave][j][t][lane] = acc[j][t];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    if (j % kWaves != wave) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4 sum = part[0][j][t][lane];
#pragma unroll
      for (int v = 1; v < kWaves; ++v) sum += part[v][j][t][lane];
      const int m = m0 + 16 * t + col;
      if (m < M) {
        bf16_t packed[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) packed[r] = f32_to_bf16(sum[r]);
        *reinterpret_cast<uint2*>(y + static_cast<int64_t>(m) * N + n0 + 16 * j + 4 * grp) =
            *reinterpret_cast<uint2*>(packed);
      }
    }
  }
}

template <bool XF32, int MT, int NTW>
hipError_t launch_mt(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  const dim3 grid(N / (16 * NTW), (M + 16 * MT - 1) / (16 * MT));
  hidden_gemm<XF32, MT, NTW><<<grid, kWaves * 64, 0, s>>>(x, static_cast<const bf16_t*>(w), static_cast<bf16_t*>(y),
                                                          M, N, K);
  return hipGetLastError();
}

// Row tiles per pass MT = 1, 2 or 4 (more rows take several passes over the weight, run
// side by side). Weight tiles per wave NTW up to MT, but no fewer than 256 workgroups
// (one per CU) over the output width: at hidden = 4096 that leaves NTW = 1.
template <bool XF32, int MT>
hipError_t launch_ntw(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  if constexpr (MT >= 4) {
    if (N % 64 == 0 && N / 64 >= kNumCUs) return launch_mt<XF32, MT, 4>(x, w, y, M, N, K, s);
  }
  if constexpr (MT >= 2) {
    if (N % 32 == 0 && N / 32 >= kNumCUs) return launch_mt<XF32, MT, 2>(x, w, y, M, N, K, s);
  }
  return launch_mt<XF32, MT, 1>(x, w, y, M, N, K, s);
}

template <bool XF32>
hipError_t launch_x(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  if (M <= 16) return launch_ntw<XF32, 1>(x, w, y, M, N, K, s);
  if (M <= 32) return launch_ntw<XF32, 2>(x, w, y, M, N, K, s);
  return launch_ntw<XF32, 4>(x, w, y, M, N, K, s);
}

// bf16 inputs, 64 weight rows per workgroup: both operands stream through LDS. The
// contraction is taken in 128-wide chunks; a chunk's stage holds the 64 weight rows and the
// 16 * MT input rows (256 bytes each), copied global -> LDS with global_load_lds_dwordx4
// (no registers held by a load in flight, whole 128-byte lines) three chunks ahead of its
// use, in a ring of four stages. Wave w multiplies weight row tile w by every input row
// tile over the whole contraction, so no partial sums need merging. In each 256-byte row
// the 16-byte pieces are stored XOR-swizzled by the row index (piece p at p ^ (row % 16)),
// so the 16 lanes that read one MFMA operand (16 rows, the same piece) hit distinct banks.
constexpr int kDmaStages = 4;
constexpr int kDmaStageBytes = 32 * 1024;   // 64 weight rows + up to 64 input rows, 256 B each
__shared__ __attribute__((aligned(16))) char g_st0[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_st1[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_st2[kDmaStageBytes];
__shared__ __attribute__((aligned(16))) char g_st3[kDmaStageBytes];
typedef __attribute__((address_space(3))) void lds_void;

template <int S>
__device__ __forceinline__ char* stage_buf() {
  static_assert(S >= 0 && S < kDmaStages, "stage");
  return S == 0 ? g_st0 : S == 1 ? g_st1 : S == 2 ? g_st2 : g_st3;
}

template <int N>
__device__ __forceinline__ void dma_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ void dma_barrier() {
  // s_barrier without __syncthreads()'s fence, which would also wait for the copies that
  // must stay in flight; callers wait for exactly the counters they need first.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MT>
__global__ __launch_bounds__(256, 1) void hidden_dma(const bf16_t* x, const bf16_t* w, bf16_t* y, int M, int N, int K) {
  constexpr int kRowsW = 64;
  constexpr int kSlotsW = kRowsW * 16;               // 16-byte slots of the weight part
  constexpr int kSlots = kSlotsW + 16 * MT * 16;     // plus the input part
  constexpr int CPW = kSlots / 64 / 4;               // copies per wave per chunk (1 KiB each)
  static_assert(CPW * 64 * 4 == kSlots && kSlots * 16 <= kDmaStageBytes, "stage layout");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * kRowsW;
  const int m0 = blockIdx.y * 16 * MT;
  const int nch = K / 128;
  const char* wbase = reinterpret_cast<const char*>(w + static_cast<int64_t>(n0) * K);
  const char* xbase = reinterpret_cast<const char*>(x + static_cast<int64_t>(m0) * K);
  // Per-lane byte offsets (within a chunk's rows) of this wave's copies; input rows past M
  // re-read row M - 1 (never stored).
  uint32_t off[CPW];
  bool is_w[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int slot = (wave * CPW + j) * 64 + lane;
    is_w[j] = (wave * CPW + j) * 64 < kSlotsW;   // uniform per copy (parts are whole KiB)
    const int part = is_w[j] ? slot : slot - kSlotsW;
    const int row = part >> 4, piece = (part & 15) ^ (row & 15);
    const int src_row = is_w[j] ? row : min(row, M - 1 - m0);
    off[j] = static_cast<uint32_t>((static_cast<int64_t>(src_row) * K + 8 * piece) * 2);
  }
  auto issue = [&](int c, char* st) {
    const int64_t kb = static_cast<int64_t>(min(c, nch - 1)) * 256;   // past the end: re-read the last chunk
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      uint32_t o = off[j];
      asm volatile("" : "+v"(o));   // a separate 32-bit operand, so the copy takes a scalar base
      const char* src = (is_w[j] ? wbase : xbase) + kb;
      __builtin_amdgcn_global_load_lds(src + o, (lds_void*)(st + (wave * CPW + j) * 1024), 16, 0, 2);
    }
  };
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Operand addresses inside a stage: weight row 16*wave + col, input row 16*t + col, piece
  // 4*ks + grp of the chunk, swizzled by the row (row % 16 == col for both).
  const int a_row = (16 * wave + col) * 256, b_row = kSlotsW * 16 + col * 256;
  auto compute = [&](const char* st) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pc = 16 * ((4 * ks + grp) ^ col);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + a_row + pc);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(st + b_row + t * 16 * 256 + pc);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  };
  // Chunk c in stage c % 4: wait for its copies (c + 1 and c + 2 may stay in flight), pass
  // the barrier that also frees stage (c + 3) % 4 (read in step c - 1), start chunk c + 3's
  // copies into it, compute.
  auto step = [&](int c, auto si) {
    constexpr int S = decltype(si)::value;
    dma_wait_vmcnt<2 * CPW>();
    dma_barrier();
    issue(c + 3, stage_buf<(S + 3) & 3>());
    compute(stage_buf<S>());
  };
  issue(0, stage_buf<0>());
  issue(1, stage_buf<1>());
  issue(2, stage_buf<2>());
  // Whole rounds of the ring, then the remaining 0-3 chunks (an exit inside an unrolled
  // round would make the compiler's wait analysis drain every copy in flight).
  const int nfull = nch & ~3;
  int c = 0;
  for (; c < nfull; c += 4) {
    step(c, std::integral_constant<int, 0>());
    step(c + 1, std::integral_constant<int, 1>());
    step(c + 2, std::integral_constant<int, 2>());
    step(c + 3, std::integral_constant<int, 3>());
  }
  if (c < nch) step(c, std::integral_constant<int, 0>());
  if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
  if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
  dma_wait_vmcnt<0>();   // the copies past the end have landed before the workgroup ends
  // D[n][m]: lane holds features n0 + 16*wave + 4*grp + r of input row m0 + 16*t + col.
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + 16 * t + col;
    if (m < M) {
      bf16_t packed[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) packed[r] = f32_to_bf16(acc[t][r]);
      *reinterpret_cast<uint2*>(y + static_cast<int64_t>(m) * N + n0 + 16 * wave + 4 * grp) =
          *reinterpret_cast<uint2*>(packed);
    }
  }
}

template <int MT>
hipError_t launch_dma(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  const dim3 grid(N / 64, (M + 16 * MT - 1) / (16 * MT));
  hidden_dma<MT><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w),
                                      static_cast<bf16_t*>(y), M, N, K);
  return hipGetLastError();
}

// bf16 inputs and a contraction in whole 256-element chunks: the 16 RT weight rows of a
// workgroup stream through an LDS ring in 512-byte runs per row (at the row stride of a wide
// layer, 256-byte runs read HBM at ~4.4 TB/s on MI355X and 512-byte runs at ~5.9), NS - 1
// chunks ahead; the inputs, which every workgroup reads (L2-resident), go straight into
// registers two chunks ahead, so LDS holds weight only. Each wave takes a quarter of every
// chunk's contraction for all the workgroup's weight rows and 16 MT input rows, and the four
// partial results are summed through LDS at the end. RT = 1, 2, 4 (16, 32, 64 rows) keeps
// about one round of workgroups on the CUs for any output width.
constexpr int kKsChunk = 256;                         // contraction per chunk (512 bytes of a row)
constexpr int kKsRingBytes = 128 * 1024;

template <int MT, int RT>
struct KsShape {
  static constexpr int kRows = 16 * RT;
  static constexpr int kStage = kRows * kKsChunk * 2;          // bytes per chunk
  static constexpr int kStages = RT == 4 ? 4 : 8;               // ring (in flight: kStages - 1)
  static constexpr int kLds = kStages * kStage;                 // 64 KiB for RT = 1: two per CU
  static constexpr int kCPW = kStage / 1024 / kWaves;          // 1 KiB copies per wave per chunk
  static constexpr int kXL = 2 * MT;                            // input loads per wave per chunk
  static constexpr int kPerCU = RT == 1 ? 2 : 1;
  static_assert(kLds <= kKsRingBytes && kCPW >= 1 && kStages % 4 == 0, "ring");
  static_assert(2 * kCPW + kXL < 64, "vmcnt range");
  static_assert(kWaves * RT * MT * 1024 <= kLds, "partials fit the ring");
};

template <int MT, int RT>
__global__ __launch_bounds__(256, (KsShape<MT, RT>::kPerCU)) void hidden_ks(const bf16_t* x, const bf16_t* w, bf16_t* y,
                                                                          int M, int N, int K) {
  using Sh = KsShape<MT, RT>;
  __shared__ __attribute__((aligned(16))) char g_ks[Sh::kLds];
  constexpr int CPW = Sh::kCPW, NS = Sh::kStages, D = NS - 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * Sh::kRows;
  const int m0 = blockIdx.y * 16 * MT;
  const int nch = K / kKsChunk;
  const char* wbase = reinterpret_cast<const char*>(w + static_cast<int64_t>(n0) * K);
  // Copy slot s of a stage holds weight row s / 32, 16-byte piece (s % 32) ^ (row % 16) of
  // the chunk's 512 bytes: the XOR spreads the 16 rows of an operand read over all banks.
  uint32_t off[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int slot = (wave * CPW + j) * 64 + lane;
    const int row = slot >> 5, piece = (slot & 31) ^ (row & 15);
    off[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) * 2u + 16u * piece;
  }
  // Input operand of tile t, step ks: row m0 + 16 t + col (rows past M re-read row M - 1 and
  // are never stored), elements 64 wave + 32 ks + 8 grp of the chunk; offsets from row m0.
  const bf16_t* xbase = x + static_cast<int64_t>(m0) * K;
  uint32_t xoff[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xoff[t] = static_cast<uint32_t>(min(16 * t + col, M - 1 - m0)) * static_cast<uint32_t>(K) + 64 * wave + 8 * grp;

  auto stage = [](int S) { return g_ks + S * Sh::kStage; };
  auto copies = [&](int c, char* st) {
    const char* src = wbase + static_cast<int64_t>(min(c, nch - 1)) * (kKsChunk * 2);   // past the end: the last chunk again
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      uint32_t o = off[j];
      asm volatile("" : "+v"(o));   // a separate 32-bit operand, so the copy takes a scalar base
      __builtin_amdgcn_global_load_lds(src + o, (lds_void*)(st + (wave * CPW + j) * 1024), 16, 0, 2);
    }
  };
  bf16x8 xb[4][MT][2];
  auto inputs = [&](int c, bf16x8 (&dst)[MT][2]) {
    const bf16_t* xc = xbase + min(c, nch - 1) * kKsChunk;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dst[t][ks] = *reinterpret_cast<const bf16x8*>(xc + xoff[t] + 32 * ks);
  };
  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const char* st, const bf16x8 (&xs)[MT][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int pc = 16 * ((8 * wave + 4 * ks + grp) ^ col);
      bf16x8 a[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) a[r] = *reinterpret_cast<const bf16x8*>(st + (16 * r + col) * (kKsChunk * 2) + pc);
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], xs[t][ks], acc[r][t], 0, 0, 0);
    }
  };
  // Issue order: weight chunk c + D follows input chunk c + 2, so waiting for the inputs of
  // chunk c leaves the copies of c + D - 2 and c + D - 1 and the inputs of c + 1 in flight
  // (chunk c's copies went out before its inputs); the barrier then also frees stage
  // (c + D) % NS, read in step c - 1.
  auto step = [&](int c, auto si) {
    constexpr int S = decltype(si)::value;
    dma_wait_vmcnt<2 * CPW + Sh::kXL>();
    dma_barrier();
    inputs(c + 2, xb[(S + 2) & 3]);
    copies(c + D, stage((S + D) % NS));
    compute(stage(S), xb[S & 3]);
  };
#pragma unroll
  for (int c = 0; c < D - 2; ++c) copies(c, stage(c));
  inputs(0, xb[0]);
  copies(D - 2, stage(D - 2));
  inputs(1, xb[1]);
  copies(D - 1, stage(D - 1));
  const int nfull = nch - nch % NS;
  int c = 0;
  for (; c < nfull; c += NS) {
    step(c, std::integral_constant<int, 0>());
    step(c + 1, std::integral_constant<int, 1>());
    step(c + 2, std::integral_constant<int, 2>());
    step(c + 3, std::integral_constant<int, 3>());
    if constexpr (NS == 8) {
      step(c + 4, std::integral_constant<int, 4>());
      step(c + 5, std::integral_constant<int, 5>());
      step(c + 6, std::integral_constant<int, 6>());
      step(c + 7, std::integral_constant<int, 7>());
    }
  }
  // The remaining 0 .. NS - 1 chunks (an exit inside an unrolled round would make the
  // compiler's wait analysis drain every load in flight).
  if (c < nch) step(c, std::integral_constant<int, 0>());
  if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>());
  if (c + 2 < nch) step(c + 2, std::integral_constant<int, 2>());
  if constexpr (NS == 8) {
    if (c + 3 < nch) step(c + 3, std::integral_constant<int, 3>());
    if (c + 4 < nch) step(c + 4, std::integral_constant<int, 4>());
    if (c + 5 < nch) step(c + 5, std::integral_constant<int, 5>());
    if (c + 6 < nch) step(c + 6, std::integral_constant<int, 6>());
  }
  dma_wait_vmcnt<0>();   // the loads past the end have landed before the ring is reused
  dma_barrier();         // every wave's last product has read its stage
  // Partials of wave q at [q][r][t][lane] (f32x4: features 16 r + 4 grp .. +4 of input row
  // 16 t + col); then each thread sums some of them over the waves.
  f32x4* red = reinterpret_cast<f32x4*>(g_ks);
  constexpr int kPart = RT * MT * 64;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave * kPart + (r * MT + t) * 64 + lane] = acc[r][t];
  __syncthreads();
  for (int e = threadIdx.x; e < kPart; e += 256) {
    f32x4 v = red[e];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) v += red[q * kPart + e];
    const int ln = e & 63, t = (e >> 6) % MT, r = (e >> 6) / MT;
    const int m = m0 + 16 * t + (ln & 15);
    if (m < M) {
      bf16_t packed[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) packed[i] = f32_to_bf16(v[i]);
      *reinterpret_cast<uint2*>(y + static_cast<int64_t>(m) * N + n0 + 16 * r + 4 * (ln >> 4)) =
          *reinterpret_cast<uint2*>(packed);
    }
  }
}

template <int MT, int RT>
hipError_t launch_ks_rt(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  const dim3 grid(N / (16 * RT), (M + 16 * MT - 1) / (16 * MT));
  hidden_ks<MT, RT><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w),
                                         static_cast<bf16_t*>(y), M, N, K);
  return hipGetLastError();
}

// Weight rows per workgroup of the 512-byte-run form for a bf16 product, 0 where another
// form is faster. Measured on MI355X (median after a 1 GiB read): 64 rows when that fills
// the CUs (16384 x 16384 at 16-64 input rows: 89-111 us against 129-153 us for the
// 256-byte-run form); 32 rows where the 256-byte-run form has under 128 workgroups
// (7168 x 16384, 64 rows: 81 against 158 us for the per-wave form), not at 8192 x 4096
// (26 against 22 us); 16 rows, two workgroups per CU, for 4096 x 4096 from 17 input rows
// (16.0 against 17.1 us at 32 rows; 10.9 against 10.1 at one row).
int ks_rows(int M, int N, int K) {
  if (K % kKsChunk != 0 || K > (1 << 20)) return 0;
  if (N % 64 == 0 && N / 64 >= kNumCUs) return 64;
  if (N % 64 == 0 && N / 64 >= kNumCUs / 2) return 0;
  if (N % 32 == 0 && N / 32 >= kNumCUs * 7 / 8) return 32;
  if (M > 16 && N % 16 == 0 && N / 16 >= kNumCUs) return 16;
  return 0;
}

template <int MT>
hipError_t launch_ks(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  switch (ks_rows(M, N, K)) {
    case 64: return launch_ks_rt<MT, 4>(x, w, y, M, N, K, s);
    case 32: return launch_ks_rt<MT, 2>(x, w, y, M, N, K, s);
    default: return launch_ks_rt<MT, 1>(x, w, y, M, N, K, s);
  }
}

// Generic: one thread per output, fp32 accumulation; any sizes, fp32 or bf16 data.
template <typename T, typename TX>
__global__ __launch_bounds__(256) void generic_hidden(const TX* x, const T* w, T* y, int M, int N, int K) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * N) return;
  const int m = static_cast<int>(i / N), n = static_cast<int>(i % N);
  float acc = 0.f;
  for (int k = 0; k < K; ++k)
    acc += Elt<TX>::load(x, static_cast<int64_t>(m) * K + k) * Elt<T>::load(w, static_cast<int64_t>(n) * K + k);
  Elt<T>::store(y, i, acc);
}

// W_fold[n][h*d_c + c] = sum_v W_O[n][h*d_v + v] W_UV^g[v][c]; one thread per element,
// threads along c (coalesced W_UV reads, W_O broadcast).
template <typename T>
__global__ __launch_bounds__(256) void fold_kernel(ProjParams d, const T* w_o, const T* w_uv, T* w_fold) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const int n = blockIdx.z;
  if (c >= d.dc) return;
  const int g = h / (d.H / d.G);
  const int64_t wo = static_cast<int64_t>(n) * d.H * d.dv + static_cast<int64_t>(h) * d.dv;
  const int64_t wu = static_cast<int64_t>(g) * d.dv * d.dc + c;
  float acc = 0.f;
  for (int v = 0; v < d.dv; ++v) acc += Elt<T>::load(w_o, wo + v) * Elt<T>::load(w_uv, wu + static_cast<int64_t>(v) * d.dc);
  Elt<T>::store(w_fold, static_cast<int64_t>(n) * d.H * d.dc + static_cast<int64_t>(h) * d.dc + c, acc);
}

}  // namespace

hipError_t launch_out_hidden(const void* x, bool x_f32, const void* w, void* y, int M, int N, int K, bool bf16,
                             hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (bf16 && !x_f32 && ks_rows(M, N, K) != 0) {
    if (M <= 16) return launch_ks<1>(x, w, y, M, N, K, s);
    if (M <= 32) return launch_ks<2>(x, w, y, M, N, K, s);
    return launch_ks<4>(x, w, y, M, N, K, s);
  }
  if (bf16 && !x_f32 && N % 64 == 0 && N / 64 >= kNumCUs / 2 && K % 128 == 0 && K <= (1 << 20)) {
    if (M <= 16) return launch_dma<1>(x, w, y, M, N, K, s);
    if (M <= 32) return launch_dma<2>(x, w, y, M, N, K, s);
    return launch_dma<4>(x, w, y, M, N, K, s);
  }
  if (bf16 && N % 16 == 0 && K % (32 * kWaves) == 0)
    return x_f32 ? launch_x<true>(x, w, y, M, N, K, s) : launch_x<false>(x, w, y, M, N, K, s);
  const int64_t n = static_cast<int64_t>(M) * N;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (bf16) {
    if (x_f32)
      generic_hidden<bf16_t, float><<<blocks, 256, 0, s>>>(static_cast<const float*>(x), static_cast<const bf16_t*>(w),
                                                           static_cast<bf16_t*>(y), M, N, K);
    else
      generic_hidden<bf16_t, bf16_t><<<blocks, 256, 0, s>>>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w),
                                                            static_cast<bf16_t*>(y), M, N, K);
  } else {
    generic_hidden<float, float><<<blocks, 256, 0, s>>>(static_cast<const float*>(x), static_cast<const float*>(w),
                                                        static_cast<float*>(y), M, N, K);
  }
  return hipGetLastError();
}

hipError_t launch_fold_out_weight(const ProjParams& p, int hidden, const void* w_o, const void* w_uv, void* w_fold,
                                  bool bf16, hipStream_t s) {
  const dim3 grid((p.dc + 255) / 256, p.H, hidden);
  if (bf16)
    fold_kernel<bf16_t><<<grid, 256, 0, s>>>(p, static_cast<const bf16_t*>(w_o), static_cast<const bf16_t*>(w_uv),
                                             static_cast<bf16_t*>(w_fold));
  else
    fold_kernel<float><<<grid, 256, 0, s>>>(p, static_cast<const float*>(w_o), static_cast<const float*>(w_uv),
                                            static_cast<float*>(w_fold));
  return hipGetLastError();
}

}  // namespace gqla
