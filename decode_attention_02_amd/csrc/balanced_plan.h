// Length-balanced split plan of the GQA decode, derived on the device.
//
// When a batch's (sequence, group) units cannot cover the CUs, the context has to be
// split; with ragged lengths, equal splits of every sequence leave the workgroups of the
// longest one with the most blocks while the others idle. Instead, the batch's blocks are
// laid end to end in sequence order and cut into `chunks` runs of
//   C = max(ceil(total / chunks), chunk_min)
// blocks; run c covers blocks [c C, (c + 1) C) and attends to one piece per sequence it meets.
// The piece of sequence b goes to partial slot c - floor(start_b / C) of b's rows, so a
// sequence of n blocks uses at most ceil(n / C) + 1 slots; the run that holds its last block
// marks the slots it does not use as empty (lse = -inf). A sequence the kernels reject (a
// length below s_q, past the block table or past the declared maximum) counts as one block:
// its one piece writes NaN partials.
#pragma once

#include "device_common.h"
#include "gqla_internal.h"

namespace gqla {

__device__ __forceinline__ int plan_blocks(const AttnParams& p, int b) {
  if (b >= p.B) return 0;
  const int L = p.ctx_lens[b];
  if (L < p.s_q || L > p.max_blocks * kBlock) return 1;
  const int n = (L + kBlock - 1) / kBlock;
  return n > p.decl_blocks ? 1 : n;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Run c: blocks [lo, hi) of the batch, run length C, the first sequence it meets (b) and
// the batch block where that sequence's blocks begin (start). Every wave computes it for
// itself from the context lengths (at most 256 sequences, 4 per lane); afterwards only these
// scalars stay live.
struct BalancedRun {
  int C, lo, hi, b, start;
  bool empty;
};

__device__ __forceinline__ BalancedRun balanced_run(const AttnParams& p, int c) {
  const int lane = threadIdx.x & 63;
  int ends[4];   // inclusive prefix of plan_blocks over sequences 64 k + lane
  int carry = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ends[k] = wave_scan(plan_blocks(p, 64 * k + lane)) + carry;
    carry = __builtin_amdgcn_readlane(ends[k], 63);
  }
  BalancedRun r;
  const int total = carry;
  r.C = max((total + p.chunks - 1) / p.chunks, p.chunk_min);
  r.lo = c * r.C;
  r.hi = min(total, r.lo + r.C);
  r.empty = r.lo >= total;
  r.b = 0;
#pragma unroll
  for (int k = 3; k >= 0; --k) {
    const uint64_t m = __ballot(64 * k + lane < p.B && ends[k] > r.lo);
    if (m != 0) r.b = 64 * k + __builtin_ctzll(m);
  }
  const int bk = r.b >> 6, bl = r.b & 63;
  const int e = bk == 0 ? __builtin_amdgcn_readlane(ends[0], bl) : bk == 1 ? __builtin_amdgcn_readlane(ends[1], bl)
              : bk == 2 ? __builtin_amdgcn_readlane(ends[2], bl) : __builtin_amdgcn_readlane(ends[3], bl);
  r.start = e - plan_blocks(p, r.b);
  // wave-uniform by construction; said so, the walk stays in scalar registers
  r.C = __builtin_amdgcn_readfirstlane(r.C);
  r.lo = __builtin_amdgcn_readfirstlane(r.lo);
  r.hi = __builtin_amdgcn_readfirstlane(r.hi);
  r.b = __builtin_amdgcn_readfirstlane(r.b);
  r.start = __builtin_amdgcn_readfirstlane(r.start);
  return r;
}

}  // namespace gqla
