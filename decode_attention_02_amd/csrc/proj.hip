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
// weight and row reads of a small batch spread over most CUs instead of a few. At large
// batches the value projection's fp32 latent outputs are the stream and get a form of their
// own (out_proj_stream: one four-wave workgroup per CU and group, each o_lat tile read once
// into an LDS ring and shared by the four waves), and so does the absorbed query
// (absorb_query_stream: the weight slice in registers, output tiles stored as whole row slices).
#include "device_common.h"
#include "gqla_internal.h"
#include "tuned.h"

#include <algorithm>
#include <type_traits>

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
// Workgroup ids are laid out so that the NZ workgroups sharing one row tile (the feature
// slices of the absorbed query, the output quarters of the value projection) have ids 8
// apart: the dispatcher places them on the same XCD at about the same time, and the rows
// they all read come from that XCD's L2 after the first. Returns (x, g, z) for a grid of
// nx * G * NZ workgroups (nx a multiple of 8).
struct GridPos {
  int x, g, z;
};
__device__ __forceinline__ GridPos grid_pos(int G, int NZ) {
  const int id = blockIdx.x, xcd = id & 7, rest = id >> 3;
  const int z = rest % NZ, r2 = rest / NZ;
  return {(r2 / G) * 8 + xcd, r2 % G, z};
}

template <int DN, int NW>
__global__ __launch_bounds__(NW * 64) void absorb_query_kernel(ProjParams d, const bf16_t* q_nope, const bf16_t* q_rope,
                                                               const bf16_t* w_uk, bf16_t* q_abs, int nx) {
  __shared__ __attribute__((aligned(16))) char w[DN * kSliceF * 2];
  constexpr int RW = 16 * NW;   // rows per workgroup pass
  const GridPos gp = grid_pos(d.G, kDC / kSliceF);
  const int g = gp.g;
  const int f0 = gp.z * kSliceF;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + RW - 1) / RW;
  if (gp.x >= n_rt) return;   // a lane of the rounded-up grid with no row tile: no copy issued
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
  for (int rt = gp.x; rt < n_rt; rt += nx) {
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
    if (gp.z == 0) {
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

// Absorbed query over many rows (large batches), where the queries and q_abs are the stream:
// workgroup (group g, latent slice z of 128 features, run of 64-row tiles). The [DN][128]
// slice of W_UK^g is staged through LDS once and read transposed into registers (the A
// operand of every tile), so a tile costs only its query loads, 8 KSA MFMAs per wave and the
// stores; the next tile's queries load under the current tile's products. Rows past the end
// re-read and re-store the last row (the same values to the same place), so every store is
// unconditional and the compiler's memory-counter waits stay exact. Each slice copies a
// quarter of the RoPE part.
template <int DN>
__global__ __launch_bounds__(256, 2) void absorb_query_stream(ProjParams d, const bf16_t* q_nope, const bf16_t* q_rope,
                                                              const bf16_t* w_uk, bf16_t* q_abs, int nx) {
  __shared__ __attribute__((aligned(16))) char w[DN * kSliceF * 2];
  constexpr int KS = DN / 32;
  constexpr int CT = kSliceF / 16;   // 16-feature output tiles of the slice
  const int nz = kDC / kSliceF;
  const int x = blockIdx.x % nx, gz = blockIdx.x / nx;
  const int g = gz / nz, z = gz % nz;
  const int f0 = z * kSliceF;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + 63) / 64;
  if (x >= n_rt) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  {
    const bf16_t* src = w_uk + static_cast<int64_t>(g) * DN * kDC + f0;
#pragma unroll
    for (int i = wave; i < DN / 4; i += 4) {
      const int r = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ swz(r);
      __builtin_amdgcn_global_load_lds(src + r * kDC + 8 * c, (lds_void*)(w + 1024 * i), 16, 0, 0);
    }
  }
  const int dq = kDC + kDR;
  auto row_of_r = [&](int rt, int r) __attribute__((always_inline)) {
    return group_row(min(rt * 64 + wave * 16 + r, rows_g - 1), g, gs, d.H);   // past the end: the last row
  };
  auto row_of = [&](int rt) __attribute__((always_inline)) { return row_of_r(rt, col); };
  auto load_q = [&](int rt, bf16x8 (&dst)[KS]) __attribute__((always_inline)) {
    const int64_t row = row_of(rt);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = *reinterpret_cast<const bf16x8*>(q_nope + row * DN + 32 * ks + 8 * grp);
  };
  bf16x8 qa[KS], qb[KS];
  load_q(x, qa);
  __builtin_amdgcn_s_waitcnt(0);   // the weight slice and the first queries have landed
  __syncthreads();
  // A operand of feature tile ct, step ks (W^T, 16 latent features x 32 nope values), read
  // transposed once: lane `col` of each 16-lane group supplies nope row 32 ks + 8 grp +
  // 4 half + (col >> 2), features 16 ct + 4 (col & 3).
  bf16x8 wa[CT][KS];
  {
    const int src_n = 8 * grp + (col >> 2);
    const int src_b = 8 * (col & 3);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r0 = 32 * ks + src_n, r1 = r0 + 4;
        const int b = 32 * ct + src_b;
        const char* p0 = w + r0 * 256 + ((((b >> 4) ^ swz(r0)) << 4) | (b & 15));
        const char* p1 = w + r1 * 256 + ((((b >> 4) ^ swz(r1)) << 4) | (b & 15));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
        wa[ct][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  }
  // Every wave has its operands before the staging area is reused for the output tiles.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  // Tile rt from the queries in `cur`; the queries of tile rt_next load into `nxt` first. Two
  // named buffers alternate (no register copy between tiles, which would wait for the loads).
  auto tile = [&](int rt, const bf16x8 (&cur)[KS], bf16x8 (&nxt)[KS], int rt_next) __attribute__((always_inline)) {
    // RoPE quarter z of the wave's 16 rows: 16 values = 32 bytes per row, two lanes per row
    // (lanes 32.. repeat lanes 0..31: the same bytes to the same place). Its load goes out
    // before the next tile's queries, so waiting for it leaves those in flight.
    const int r16 = (lane & 31) >> 1, half = lane & 1;
    const int64_t orow = group_row(min(rt * 64 + wave * 16 + r16, rows_g - 1), g, gs, d.H);
    const uint4 rope = *reinterpret_cast<const uint4*>(q_rope + orow * kDR + 16 * z + 8 * half);
    load_q(min(rt_next, n_rt - 1), nxt);   // past the last tile: the last tile again
    __builtin_amdgcn_sched_barrier(0);
    // The tile's 16 rows x 128 features go through this wave's 4 KiB of the (now free) weight
    // staging area, so the stores are whole 256-byte row slices (16 bytes per lane) instead of
    // 8-byte pieces: row r's 16-byte chunk c sits at chunk c ^ (r & 15) of its LDS row.
    char* stage = w + wave * 4096;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ct][ks], cur[ks], acc, 0, 0, 0);
      bf16_t packed[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[k]);
      // Lane (row col, grp) holds features 16 ct + 4 grp .. +4: half of 16-byte chunk 2 ct + grp / 2.
      const int c = 2 * ct + (grp >> 1);
      *reinterpret_cast<uint2*>(stage + col * 256 + 16 * (c ^ col) + 8 * (grp & 1)) = *reinterpret_cast<uint2*>(packed);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * k + (lane >> 4), c = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * 256 + 16 * (c ^ r));
      const int64_t orr = row_of_r(rt, r);
      *reinterpret_cast<uint4*>(q_abs + orr * dq + f0 + 8 * c) = v;
    }
    *reinterpret_cast<uint4*>(q_abs + orow * dq + kDC + 16 * z + 8 * half) = rope;
  };
  const int nt = (n_rt - x + nx - 1) / nx;   // tiles x, x + nx, ... of this workgroup
  int j = 0;
  for (; j + 2 <= nt; j += 2) {
    tile(x + j * nx, qa, qb, x + (j + 1) * nx);
    tile(x + (j + 1) * nx, qb, qa, x + (j + 2) * nx);
  }
  if (j < nt) tile(x + j * nx, qa, qb, x + (j + 1) * nx);
  __builtin_amdgcn_s_waitcnt(0);   // the loads past the end have landed before the workgroup ends
}

__global__ __launch_bounds__(64) void out_proj_kernel(ProjParams d, const float* o_lat, const bf16_t* w_uv, bf16_t* out,
                                                      int nx) {
  const GridPos gp = grid_pos(d.G, kDV / 32);
  const int g = gp.g;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + 15) / 16;
  if (gp.x >= n_rt) return;   // a lane of the rounded-up grid with no row tile
  const int lane = threadIdx.x, wave = gp.z;   // one wave per workgroup: its 32 rows of W_UV^g
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
  for (int rt = gp.x; rt < n_rt; rt += nx) {
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

// Value projection over many rows (large batches), where the latent outputs are the
// stream: one workgroup per (group, run of 16-row tiles), its four waves holding W_UV^g rows
// 32w .. +32 in registers and sharing each tile of o_lat, which goes through an LDS ring
// (global_load_lds, three tiles ahead). Every latent output is then read from memory once,
// instead of once per 32 output features by the single-wave form.
constexpr int kOpTileBytes = 16 * kDC * 4;             // 16 rows of fp32 o_lat: 32 KiB
constexpr int kOpCPW = kOpTileBytes / 1024 / 4;        // 1 KiB copies per wave per tile (8)

template <int N>
__device__ __forceinline__ void op_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ void op_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256, 1) void out_proj_stream(ProjParams d, const float* o_lat, const bf16_t* w_uv,
                                                          bf16_t* out, int nx) {
  // One array per stage: the compiler then sees that the copies into one stage do not
  // alias the reads of another, and waits only for the copies it must.
  __shared__ __attribute__((aligned(16))) char ring0[kOpTileBytes];
  __shared__ __attribute__((aligned(16))) char ring1[kOpTileBytes];
  __shared__ __attribute__((aligned(16))) char ring2[kOpTileBytes];
  __shared__ __attribute__((aligned(16))) char hl[2][16 * kDC * 2];   // bf16 high / low parts of one tile
  const int g = blockIdx.x / nx, x = blockIdx.x % nx;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int n_rt = (rows_g + 15) / 16;
  if (x >= n_rt) return;
  const int nt = (n_rt - x + nx - 1) / nx;   // tiles x, x + nx, ... of this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 wa[2][kDC / 32];
  {
    const bf16_t* wsrc = w_uv + (static_cast<int64_t>(g) * kDV + 32 * wave + col) * kDC + 8 * grp;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < kDC / 32; ++ks) wa[t][ks] = *reinterpret_cast<const bf16x8*>(wsrc + 16 * t * kDC + 32 * ks);
  }
  auto stage = [&](int S) __attribute__((always_inline)) { return S == 0 ? ring0 : S == 1 ? ring1 : ring2; };
  // Copy j of a wave fills 16-byte chunks (8 wave + j) * 64 + lane of the tile: row
  // (8 wave + j) / 2 (the same for the whole wave), position p = 64 ((8 wave + j) % 2) + lane
  // of its 128 chunks, which holds source chunk p ^ row (rows 0..15).
  auto copies = [&](int j, char* st) __attribute__((always_inline)) {
    const int rt = x + min(j, nt - 1) * nx;   // past the end: the last tile again
#pragma unroll
    for (int k = 0; k < kOpCPW; ++k) {
      const int c = wave * kOpCPW + k;
      const int row = c >> 1;
      const int rg = min(rt * 16 + row, rows_g - 1);
      const float* src = o_lat + group_row(rg, g, gs, d.H) * kDC;
      uint32_t off = 16u * static_cast<uint32_t>((64 * (c & 1) + lane) ^ row);
      asm volatile("" : "+v"(off));   // a separate 32-bit operand, so the copy takes a scalar base
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off, (lds_void*)(st + c * 1024), 16, 0, 2);
    }
  };
  // Wave w splits rows 4w .. 4w + 3 of the tile into bf16 high and low parts, once for all
  // four waves: lane l takes row 4w + l / 16 and its 8-value chunks c = l % 16 + 16 q. Chunk c
  // of row r is stored at chunk c ^ r of the row in `hl`, so the 16 rows of an operand read
  // sit in 16 different bank groups.
  auto split = [&](const char* st) __attribute__((always_inline)) {
    const int r = 4 * wave + (lane >> 4);
    f32x4 xs[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = (lane & 15) + 16 * q;
      xs[q][0] = *reinterpret_cast<const f32x4*>(st + r * (kDC * 4) + 16 * ((2 * c) ^ r));
      xs[q][1] = *reinterpret_cast<const f32x4*>(st + r * (kDC * 4) + 16 * ((2 * c + 1) ^ r));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = (lane & 15) + 16 * q;
      const f32x4 x0 = xs[q][0], x1 = xs[q][1];
      bf16x8 hi, lo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v = k < 4 ? x0[k] : x1[k - 4];
        const __bf16 h = static_cast<__bf16>(v);
        hi[k] = h;
        lo[k] = static_cast<__bf16>(v - static_cast<float>(h));
      }
      *reinterpret_cast<bf16x8*>(hl[0] + r * (kDC * 2) + 16 * (c ^ r)) = hi;
      *reinterpret_cast<bf16x8*>(hl[1] + r * (kDC * 2) + 16 * (c ^ r)) = lo;
    }
  };
  auto compute = [&](int j) __attribute__((always_inline)) {
    // All operands are read first: with copies in flight the compiler can only wait for the
    // LDS counter to drain, so reads issued step by step would each wait a full round trip.
    bf16x8 hs[kDC / 32], ls[kDC / 32];
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks) {
      const int o = col * (kDC * 2) + 16 * ((4 * ks + grp) ^ col);
      hs[ks] = *reinterpret_cast<const bf16x8*>(hl[0] + o);
      ls[ks] = *reinterpret_cast<const bf16x8*>(hl[1] + o);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks) {
      const bf16x8 hi = hs[ks], lo = ls[ks];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[t][ks], hi, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[t][ks], lo, acc[t], 0, 0, 0);
      }
    }
    const int rg = (x + j * nx) * 16 + col;
    if (rg < rows_g) {
      const int64_t orow = group_row(rg, g, gs, d.H);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16_t packed[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[t][k]);
        *reinterpret_cast<uint2*>(out + orow * kDV + 32 * wave + 16 * t + 4 * grp) = *reinterpret_cast<uint2*>(packed);
      }
    }
  };
  // Tile j in stage j % 3: wait for its copies (j + 1 may stay in flight; the weight loads
  // went out first), pass the barrier that also frees stage (j + 2) % 3 (split in step
  // j - 1) and the split buffer (read in step j - 1), start tile j + 2's copies, split,
  // pass the second barrier, compute.
  auto step = [&](int j, auto si) __attribute__((always_inline)) {
    constexpr int S = decltype(si)::value;
    op_wait_vmcnt<kOpCPW>();
    op_barrier();
    copies(j + 2, stage((S + 2) % 3));
    split(stage(S));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    op_barrier();
    compute(j);
  };
  copies(0, stage(0));
  copies(1, stage(1));
  const int nfull = nt - nt % 3;
  int j = 0;
  for (; j < nfull; j += 3) {
    step(j, std::integral_constant<int, 0>());
    step(j + 1, std::integral_constant<int, 1>());
    step(j + 2, std::integral_constant<int, 2>());
  }
  if (j < nt) step(j, std::integral_constant<int, 0>());
  if (j + 1 < nt) step(j + 1, std::integral_constant<int, 1>());
  op_wait_vmcnt<0>();   // the copies past the end have landed before the workgroup ends
}

// Split combine fused with the value projection (absorb path, split decode). Workgroup
// (row tile of R rows of group g, g) merges its rows' split partials,
//   o = sum_s w_s o_s / sum_s w_s,  w_s = exp(lse_s - max lse),
// writes them to o_lat (and lse), keeps them in LDS as bf16 high and low parts, and applies
// W_UV^g to them: wave w takes W_UV^g rows 32w .. +32 (two 16-row MFMA tiles, A from global
// memory) against the 16 MFMA columns (B from LDS; columns R .. 15 are zero when R < 16).
// One launch instead of the combine and the value projection, and the merged rows are read
// back from LDS instead of memory. R < 16 gives small batches enough workgroups: the merge
// is a latency-bound read of the partials, and 64 workgroups leave most CUs idle.
constexpr int kCombMaxSplits = 64;
constexpr int kCombPad = kDC + 8;   // LDS row stride in bf16: rows start 16 bytes apart in the banks

template <int R>
__global__ __launch_bounds__(256) void combine_out_proj_kernel(ProjParams d, const float* ws_o, const float* ws_lse,
                                                               int n_split, float* o_lat, float* lse_out,
                                                               const bf16_t* w_uv, bf16_t* out) {
  constexpr int T = 256 / R;       // threads per row
  constexpr int C = kDC / 4 / T;   // float4 columns per thread and split
  constexpr int U = 16 / C;        // splits per pass: 16 float4 loads in flight per thread
  static_assert(R == 4 || R == 8 || R == 16, "row tile");
  __shared__ float s_w[R][kCombMaxSplits];
  __shared__ float s_inv[R];
  __shared__ __attribute__((aligned(16))) bf16_t s_hi[16][kCombPad];
  __shared__ __attribute__((aligned(16))) bf16_t s_lo[16][kCombPad];
  const int g = blockIdx.y;
  const int gs = d.H / d.G;
  const int rows_g = d.rows * gs;
  const int rg0 = blockIdx.x * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid / T, j = tid % T;
  const int rg = rg0 + r;
  const bool live = rg < rows_g;
  const int64_t row = live ? group_row(rg, g, gs, d.H) : 0;
  // This wave's 32 rows of W_UV^g as MFMA A operands (wave w, rows 32 w + 16 t + col, 8
  // latent values from 32 ks + 8 grp), loaded first so that they arrive under the merge.
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 wa[kDC / 32][2];
  {
    const bf16_t* wsrc = w_uv + (static_cast<int64_t>(g) * kDV + 32 * wave + col) * kDC + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) wa[ks][t] = *reinterpret_cast<const bf16x8*>(wsrc + 16 * t * kDC + 32 * ks);
  }
  // Weights: T threads per row, each over every T-th split, then a reduction over the T.
  {
    const float* lse = ws_lse + row * n_split;
    float m = -INFINITY;
    bool nan = false;
    for (int sp = j; sp < n_split; sp += T) {
      const float l = live ? lse[sp] : -INFINITY;
      nan |= l != l;
      m = fmaxf(m, l);
    }
    for (int o = T / 2; o > 0; o >>= 1) {
      m = fmaxf(m, __shfl_xor(m, o, T));
      nan |= __shfl_xor(static_cast<int>(nan), o, T) != 0;
    }
    float tot = 0.f;
    for (int sp = j; sp < n_split; sp += T) {
      const float l = live ? lse[sp] : -INFINITY;
      const float w = (l == -INFINITY) ? 0.f : expf(l - m);
      s_w[r][sp] = w;
      tot += w;
    }
    for (int o = T / 2; o > 0; o >>= 1) tot += __shfl_xor(tot, o, T);
    const bool nan_row = nan || !(tot > 0.f);
    if (j == 0) {
      s_inv[r] = live ? (nan_row ? nan_f32() : 1.f / tot) : 0.f;
      if (live && lse_out != nullptr) lse_out[row] = nan_row ? nan_f32() : m + logf(tot);
    }
  }
  if constexpr (R < 16) {   // the unused MFMA columns
    for (int i = tid; i < (16 - R) * kCombPad / 8; i += 256) {
      const int rr = R + i / (kCombPad / 8), c = 8 * (i % (kCombPad / 8));
      *reinterpret_cast<uint4*>(&s_hi[rr][c]) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&s_lo[rr][c]) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  // Merge: thread (row r, j) takes the float4 columns j + T k (k < C) of the row's 512
  // features, so the T threads of a row read 16 T contiguous bytes per k. U splits per
  // pass, their loads issued before the first product, so a thread waits about once per
  // U splits instead of once per split.
  {
    const float* src = ws_o + row * n_split * kDC;
    float4 acc[C];
#pragma unroll
    for (int k = 0; k < C; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
      for (int sp0 = 0; sp0 < n_split; sp0 += U) {
        float w[U];
        float4 v[U][C];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          w[u] = sp0 + u < n_split ? s_w[r][sp0 + u] : 0.f;
          const float* o = src + static_cast<int64_t>(sp0 + u) * kDC;
          // an empty split (weight 0, uniform over the row): its partials are not read
#pragma unroll
          for (int k = 0; k < C; ++k)
            v[u][k] = w[u] != 0.f ? *reinterpret_cast<const float4*>(o + 4 * (j + T * k)) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < C; ++k) {
            acc[k].x += w[u] * v[u][k].x; acc[k].y += w[u] * v[u][k].y;
            acc[k].z += w[u] * v[u][k].z; acc[k].w += w[u] * v[u][k].w;
          }
      }
    }
    const float inv = s_inv[r];
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const int f = 4 * (j + T * k);   // first of the 4 features
      const float x[4] = {acc[k].x * inv, acc[k].y * inv, acc[k].z * inv, acc[k].w * inv};
      if (live) *reinterpret_cast<float4*>(o_lat + row * kDC + f) = make_float4(x[0], x[1], x[2], x[3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 h = static_cast<__bf16>(x[e]);
        s_hi[r][f + e] = __builtin_bit_cast(bf16_t, h);
        s_lo[r][f + e] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(x[e] - static_cast<float>(h)));
      }
    }
  }
  __syncthreads();
  // out^T = W_UV^g o^T: B = 8 latent values of row col.
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < kDC / 32; ++ks) {
    const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&s_hi[col][32 * ks + 8 * grp]);
    const bf16x8 lo = *reinterpret_cast<const bf16x8*>(&s_lo[col][32 * ks + 8 * grp]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks][t], hi, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks][t], lo, acc[t], 0, 0, 0);
    }
  }
  const int rgc = rg0 + col;
  if (col < R && rgc < rows_g) {
    const int64_t orow = group_row(rgc, g, gs, d.H);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16_t packed[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) packed[k] = f32_to_bf16(acc[t][k]);
      *reinterpret_cast<uint2*>(out + orow * kDV + 32 * wave + 16 * t + 4 * grp) = *reinterpret_cast<uint2*>(packed);
    }
  }
}

// Row tile of the fused combine: the largest of 16, 8, 4 rows that still gives at least
// 256 workgroups (one per CU), else 4.
int comb_rows(int rows_g, int G) {
  for (int R = 16; R > 4; R /= 2)
    if (static_cast<int64_t>((rows_g + R - 1) / R) * G >= 256) return R;
  return 4;
}

}  // namespace

bool tuned_combine_out_supported(const gqla_dims* d, int n_split) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->v_dim == kDV && n_split > 1 && n_split <= kCombMaxSplits;
}

hipError_t launch_tuned_combine_out(const ProjParams& p, const float* ws_o, const float* ws_lse, int n_split,
                                    float* o_lat, float* lse, const void* w_uv, void* out, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  const int R = comb_rows(rows_g, p.G);
  const dim3 grid((rows_g + R - 1) / R, p.G);
  const bf16_t* wv = static_cast<const bf16_t*>(w_uv);
  bf16_t* o = static_cast<bf16_t*>(out);
  if (R == 16)
    combine_out_proj_kernel<16><<<grid, 256, 0, s>>>(p, ws_o, ws_lse, n_split, o_lat, lse, wv, o);
  else if (R == 8)
    combine_out_proj_kernel<8><<<grid, 256, 0, s>>>(p, ws_o, ws_lse, n_split, o_lat, lse, wv, o);
  else
    combine_out_proj_kernel<4><<<grid, 256, 0, s>>>(p, ws_o, ws_lse, n_split, o_lat, lse, wv, o);
  return hipGetLastError();
}

bool tuned_absorb_query_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->rope_dim == kDR &&
         (d->nope_dim == 64 || d->nope_dim == 128);
}

hipError_t launch_tuned_absorb_query(const ProjParams& p, const void* q_nope, const void* q_rope, const void* w_uk,
                                     void* q_abs, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  const int per_row = (kDC / kSliceF) * p.G;
  {
    // Many rows: about two workgroups per CU, each streaming at least 16 tiles of 64 rows.
    const int n_rt64 = (rows_g + 63) / 64;
    const int nx = std::max(1, 2 * kNumCUs / per_row);
    if (n_rt64 >= 16 * nx) {
      const bf16_t* qn = static_cast<const bf16_t*>(q_nope);
      const bf16_t* qr = static_cast<const bf16_t*>(q_rope);
      const bf16_t* wk = static_cast<const bf16_t*>(w_uk);
      bf16_t* qa = static_cast<bf16_t*>(q_abs);
      const dim3 grid(static_cast<unsigned>(nx * per_row));
      if (p.dn == 128) absorb_query_stream<128><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa, nx);
      else absorb_query_stream<64><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa, nx);
      return hipGetLastError();
    }
  }
  const bool wide = static_cast<int64_t>((rows_g + 63) / 64) * per_row >= kNumCUs;
  const int n_rt = wide ? (rows_g + 63) / 64 : (rows_g + 15) / 16;
  const int nx = (std::max(1, std::min(n_rt, kMaxWGs / per_row)) + 7) / 8 * 8;   // row-tile lanes, x8 for grid_pos
  const int64_t wgs = static_cast<int64_t>(nx) * per_row;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(wgs));
  const bf16_t* qn = static_cast<const bf16_t*>(q_nope);
  const bf16_t* qr = static_cast<const bf16_t*>(q_rope);
  const bf16_t* wk = static_cast<const bf16_t*>(w_uk);
  bf16_t* qa = static_cast<bf16_t*>(q_abs);
  if (wide) {
    if (p.dn == 128) absorb_query_kernel<128, 4><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa, nx);
    else absorb_query_kernel<64, 4><<<grid, 256, 0, s>>>(p, qn, qr, wk, qa, nx);
  } else {
    if (p.dn == 128) absorb_query_kernel<128, 1><<<grid, 64, 0, s>>>(p, qn, qr, wk, qa, nx);
    else absorb_query_kernel<64, 1><<<grid, 64, 0, s>>>(p, qn, qr, wk, qa, nx);
  }
  return hipGetLastError();
}

bool tuned_out_proj_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->v_dim == kDV;
}

hipError_t launch_tuned_out_proj(const ProjParams& p, const float* o_lat, const void* w_uv, void* out, hipStream_t s) {
  const int rows_g = p.rows * (p.H / p.G);
  const int n_rt = (rows_g + 15) / 16;
  // Many rows: four-wave workgroups sharing each o_lat tile through LDS, about one per CU,
  // each with at least 8 tiles (the weight load is then small next to the stream).
  const int nx_stream = std::max(1, kNumCUs / p.G);
  if (n_rt >= 8 * nx_stream) {
    out_proj_stream<<<static_cast<unsigned>(nx_stream * p.G), 256, 0, s>>>(p, o_lat, static_cast<const bf16_t*>(w_uv),
                                                                           static_cast<bf16_t*>(out), nx_stream);
    return hipGetLastError();
  }
  // One wave per workgroup (32 rows of W_UV^g, z = which 32), so that the weight and
  // latent-output reads spread over many CUs. Each wave loads its 32 KiB of W_UV^g once;
  // with many row tiles a wave visits at least 4 of them so that weight reloads stay small
  // next to the latent-output reads.
  const int want = std::max((n_rt + 3) / 4, 256 / p.G);
  const int nx = (std::max(1, std::min({n_rt, want, kMaxWGs / p.G})) + 7) / 8 * 8;   // x8 for grid_pos
  const int64_t wgs = static_cast<int64_t>(nx) * p.G * (kDV / 32);
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  out_proj_kernel<<<static_cast<unsigned>(wgs), 64, 0, s>>>(p, o_lat, static_cast<const bf16_t*>(w_uv),
                                                            static_cast<bf16_t*>(out), nx);
  return hipGetLastError();
}

}  // namespace gqla
