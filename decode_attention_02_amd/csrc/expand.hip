// Latent -> per-group K/V cache expansion on gfx950 MFMA (bf16, fp32 accumulation).
//
// GQLA's GQA path expands the cached latent into G full key/value heads ("GQLA:
// Attention latente ...", English abstract; gqla_attn.py docstring, GQA path):
//   K[p][g][r] = [ W_UK^g c_r ; kr_r ],  V[p][g][r] = W_UV^g c_r,
// a GEMM of 64-token latent tiles against each group's stacked [W_UK^g ; W_UV^g]
// (d_n + d_v rows by d_c = 512).
//
// A workgroup owns one group and a run of listed blocks. Each wave keeps a 32-row
// slice of [W_UK^g ; W_UV^g] in registers for the whole run, so the weights are read
// once per workgroup, while the latent tiles stream through LDS (global_load_lds,
// double-buffered, the XOR-swizzled layout of the absorb decode). Key rows come out of
// K^T = W_UK^g C^T, whose accumulator holds 4 consecutive key features of one token; value
// rows come out of V = C W_UV^g^T, whose accumulator holds 4 consecutive tokens of one
// feature. Two such accumulators (two feature tiles of a key, two token tiles of a value)
// are paired across lane rows with v_permlane16_swap so that each lane stores 16 contiguous
// bytes. The RoPE key is copied into every group's K.
#include "device_common.h"
#include "gqla_internal.h"
#include "tuned.h"

#include <algorithm>

namespace gqla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kDQ = kDC + kDR;
constexpr int kRowBytes = kDQ * 2;
constexpr int kChunks = kDQ / 8;
constexpr int kTileBytes = kBlock * kRowBytes;
constexpr int kDV = 128;

// Chunk swizzle of the latent tile in LDS: chunk c of token row t sits at c xor swz(t)
// inside its 8-chunk group, swz(t) = 2 (t0 xor t3) + 4 t1, the absorb decode's layout. Chosen
// by measurement: against (t mod 8) xor t3 the expansion is 1.5-4% faster at 8 and 16 groups
// (same bits out; the operand reads take one chunk of each of 16 rows).
__device__ __forceinline__ int swz(int t) { return 2 * ((t ^ (t >> 3)) & 1) + 4 * ((t >> 1) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The expanded cache is written once here and read by later decode calls, not by this
// kernel: non-temporal 16-byte stores (6.6-8% faster at 16 groups, 0-6% at 8, no change at
// 2, than ordinary stores; the same bytes).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(bf16_t* dst, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane l's bytes
// land at lds + 16 * l.
__device__ __forceinline__ void copy16_to_lds(const char* g, lds_void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

__shared__ __attribute__((aligned(16))) char e_tile0[kTileBytes];
__shared__ __attribute__((aligned(16))) char e_tile1[kTileBytes];
constexpr int kMaxRun = 2048;        // listed blocks per workgroup (ids staged in LDS)
__shared__ int32_t e_ids[kMaxRun];

template <int BUF>
__device__ __forceinline__ char* etile() { return BUF == 0 ? e_tile0 : e_tile1; }

// DN = nope dim (64 or 128); W = (DN + 128) / 32 waves, wave w owns stacked weight rows
// 32w .. 32w+31 (key rows first, then value rows).
template <int DN>
struct ExpandCta {
  static constexpr int DQK = DN + kDR;
  static constexpr int W = (DN + kDV) / 32;
  static constexpr int PER_WAVE = kChunks * kBlock / 64 / W;
  static_assert(PER_WAVE * W * 64 == kChunks * kBlock, "tile must split evenly over waves");
  static constexpr int KS = kDC / 32;

  const ProjParams& d;
  const bf16_t* latent;
  const int32_t* ids;
  int64_t num_blocks;
  bf16_t* expanded;
  int g, j0, nj;
  int lane, wave, col, grp;
  bool is_key;
  ExpandedLayout lay;   // this cache's block layout (RoPE key per group or shared)
  int k_feats;          // K features stored in each group chunk
  int row0;                 // first weight row of this wave within its matrix
  bf16x8 wf[2][KS];         // the wave's weight rows, MFMA operand layout
  int base_even, base_odd;  // per-lane LDS offsets of the latent operand
  int dma_off[PER_WAVE];    // per-lane source offsets of the tile copy

  __device__ ExpandCta(const ProjParams& d_, const bf16_t* lat, const int32_t* ids_, int64_t nb, bf16_t* ex)
      : d(d_), latent(lat), ids(ids_), num_blocks(nb), expanded(ex) {}

  // Ids staged in LDS (-1 = outside the pool, skipped), so fetching one never waits on
  // the vector-memory counter that tracks the tile copies.
  __device__ __forceinline__ int block_id(int j) const { return e_ids[j]; }

  template <int BUF>
  __device__ __forceinline__ void issue(int j) {
    const int id = max(block_id(j), 0);   // skipped ids still copy a valid block
    const char* src = reinterpret_cast<const char*>(latent) + static_cast<int64_t>(id) * kTileBytes;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k)
      copy16_to_lds(src + dma_off[k], (lds_void*)(etile<BUF>() + (wave * PER_WAVE + k) * 1024));
  }

  // Two 8-byte halves (4 bf16 each, in lanes of rows 2m and 2m + 1 of the wave) become one
  // 16-byte piece per lane: v_permlane16_swap exchanges `a` of the odd rows with `b` of the
  // even rows, so even-row lanes end with (a of row 2m, a of row 2m + 1) and odd-row lanes
  // with (b of row 2m, b of row 2m + 1).
  __device__ __forceinline__ static uint4 pair16(const f32x4& a, const f32x4& b) {
    bf16_t pa[4], pb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) { pa[k] = f32_to_bf16(a[k]); pb[k] = f32_to_bf16(b[k]); }
    const uint2 ua = *reinterpret_cast<const uint2*>(pa), ub = *reinterpret_cast<const uint2*>(pb);
    const auto x = __builtin_amdgcn_permlane16_swap(ua.x, ub.x, false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(ua.y, ub.y, false, false);
    return uint4{x[0], y[0], x[1], y[1]};
  }

  // Key rows (K^T = W C^T) or value rows (V = C W^T) of one 64-token tile, two 16-token
  // tiles at a time; the orientation is a compile-time choice taken under a wave-uniform
  // branch. Every store is a 16-byte piece: 16 lanes x 64 bytes of contiguous slab rows
  // (keys) or 64 bytes of a value row per lane group (values).
  template <int BUF, bool KEY>
  __device__ __forceinline__ void tiles(bf16_t* chunk) {
    const char* tile = etile<BUF>();
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      f32x4 acc[2][2];   // [16-token tile 2 hp + u][ft]
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) acc[u][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto ld = [&](int u, int ks) {
        const char* rows = tile + (2 * hp + u) * 16 * kRowBytes;
        return *reinterpret_cast<const bf16x8*>(rows + ((ks & 1) ? base_odd : base_even) + 128 * (ks >> 1));
      };
      bf16x8 a0[2] = {ld(0, 0), ld(1, 0)}, a1[2] = {ld(0, 1), ld(1, 1)};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 a2[2] = {a1[0], a1[1]};
        if (ks + 2 < KS) { a2[0] = ld(0, ks + 2); a2[1] = ld(1, ks + 2); }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int ft = 0; ft < 2; ++ft) {
            if (KEY) acc[u][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ft][ks], a0[u], acc[u][ft], 0, 0, 0);
            else acc[u][ft] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[u], wf[ft][ks], acc[u][ft], 0, 0, 0);
          }
#pragma unroll
        for (int u = 0; u < 2; ++u) { a0[u] = a1[u]; a1[u] = a2[u]; }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Offset of a lane's 16 bytes inside its 32-value run: 16 (grp & 1) + 8 (grp >> 1) values.
      const int off = 16 * (grp & 1) + 8 * (grp >> 1);
      if (KEY) {
        // K^T tile u: lane = token 16 (2 hp + u) + col; ft 0 / 1 hold key features
        // row0 + 4 grp / row0 + 16 + 4 grp (.. +4) of the 32-feature slab row0 / 32.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 v = pair16(acc[u][0], acc[u][1]);
          const int tok = (2 * hp + u) * 16 + col;
          store_stream(chunk + (row0 / kSlab) * kBlock * kSlab + tok * kSlab + off, v);
        }
      } else {
        // V tile u: lane = value feature row0 + 16 ft + col, tokens 32 hp + 16 u + 4 grp (.. +4)
        // of the 32-token half hp.
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) {
          const uint4 v = pair16(acc[0][ft], acc[1][ft]);
          const int f = row0 + 16 * ft + col;
          store_stream(chunk + kBlock * k_feats + hp * kDV * kHalf + f * kHalf + off, v);
        }
      }
    }
  }

  template <int BUF>
  __device__ __forceinline__ void compute(int id) {
    const char* tile = etile<BUF>();
    bf16_t* blk = expanded + static_cast<int64_t>(id) * lay.block;
    bf16_t* chunk = blk + lay.rope + g * lay.chunk;
    if (is_key) tiles<BUF, true>(chunk);
    else tiles<BUF, false>(chunk);
    // RoPE key copy: 64 tokens x 64 values, 16 bytes per lane-step over the workgroup; into
    // every group's K, or once per block into the shared key area.
    if (d.rope_shared && g != 0) return;
    bf16_t* kdst = d.rope_shared ? blk : chunk;
    const int kf0 = d.rope_shared ? 0 : DN;
    for (int i = threadIdx.x; i < kBlock * kDR / 8; i += W * 64) {
      const int tok = i / (kDR / 8), c = kDC / 8 + i % (kDR / 8);
      const uint4 v = *reinterpret_cast<const uint4*>(tile + tok * kRowBytes + (((c & ~7) | ((c & 7) ^ swz(tok))) << 4));
      const int fk = kf0 + 8 * (i % (kDR / 8));
      store_stream(kdst + (fk / kSlab) * kBlock * kSlab + tok * kSlab + fk % kSlab, v);
    }
  }

  template <int BUF>
  __device__ __forceinline__ void step(int j) {
    issue<1 - BUF>(min(j + 1, nj - 1));
    wait_vmcnt<PER_WAVE>();
    lds_barrier();
    if (j < nj) {
      const int id = block_id(j);
      if (id >= 0) compute<BUF>(id);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
  }

  __device__ __forceinline__ void run(const bf16_t* w_uk, const bf16_t* w_uv, int j0_, int nj_, int g_) {
    j0 = j0_;
    nj = nj_;
    g = g_;
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    col = lane & 15;
    grp = lane >> 4;
    lay = expanded_layout(DN, kDR, kDV, d.G, d.rope_shared != 0);
    k_feats = lay.k_feats;
    is_key = wave * 32 < DN;
    row0 = is_key ? wave * 32 : wave * 32 - DN;
    const bf16_t* wmat = is_key ? w_uk + static_cast<int64_t>(g) * DN * kDC : w_uv + static_cast<int64_t>(g) * kDV * kDC;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        wf[ft][ks] = *reinterpret_cast<const bf16x8*>(wmat + static_cast<int64_t>(row0 + 16 * ft + col) * kDC + 32 * ks + 8 * grp);
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int slot = (wave * PER_WAVE + k) * 64 + lane;
      const int t = slot / kChunks, cp = slot - t * kChunks;
      dma_off[k] = t * kRowBytes + 16 * ((cp & ~7) | ((cp & 7) ^ swz(t)));
    }
    {
      const int sw = swz(col);
      const int lo2 = (grp ^ sw) & 3;
      base_even = col * kRowBytes + 16 * ((0 ^ (sw & 4)) | lo2);
      base_odd = col * kRowBytes + 16 * ((4 ^ (sw & 4)) | lo2);
    }
    for (int i = threadIdx.x; i < nj; i += W * 64) {
      const int32_t id = ids[j0 + i];
      e_ids[i] = (id < 0 || id >= num_blocks) ? -1 : id;
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    lds_barrier();
    issue<0>(0);
    for (int j = 0; j < nj; j += 2) {
      step<0>(j);
      step<1>(j + 1);
    }
    wait_vmcnt<0>();
  }
};

template <int DN>
__global__ __launch_bounds__((DN + kDV) / 32 * 64, 1) void expand_blocks(ProjParams d, const bf16_t* latent, const bf16_t* w_uk,
                                                                         const bf16_t* w_uv, const int32_t* ids, int64_t n_ids,
                                                                         int64_t num_blocks, int per_wg, bf16_t* expanded) {
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * per_wg;
  const int nj = static_cast<int>(min<int64_t>(per_wg, n_ids - j0));
  if (nj <= 0) return;
  ExpandCta<DN> cta(d, latent, ids, num_blocks, expanded);
  cta.run(w_uk, w_uv, static_cast<int>(j0), nj, blockIdx.y);
}

}  // namespace

bool tuned_expand_supported(const gqla_dims* d) {
  return d->dtype == GQLA_BF16 && d->latent_rank == kDC && d->rope_dim == kDR && d->v_dim == kDV &&
         (d->nope_dim == 64 || d->nope_dim == 128);
}

hipError_t launch_tuned_expand(const ProjParams& p, const void* latent, const void* w_uk, const void* w_uv,
                               const int32_t* block_ids, int64_t n_blocks, int64_t num_blocks, void* expanded,
                               hipStream_t s) {
  // Enough workgroups to cover the CUs, each holding its group's weights for a run of blocks.
  const int64_t per_group = std::max<int64_t>(1, (2 * kNumCUs + p.G - 1) / p.G);
  const int per_wg = static_cast<int>(std::min<int64_t>(kMaxRun, std::max<int64_t>(1, (n_blocks + per_group - 1) / per_group)));
  const int64_t wgs = (n_blocks + per_wg - 1) / per_wg;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(wgs), p.G);
  const bf16_t* lat = static_cast<const bf16_t*>(latent);
  const bf16_t* wk = static_cast<const bf16_t*>(w_uk);
  const bf16_t* wv = static_cast<const bf16_t*>(w_uv);
  bf16_t* ex = static_cast<bf16_t*>(expanded);
  if (p.dn == 128)
    expand_blocks<128><<<grid, (128 + kDV) / 32 * 64, 0, s>>>(p, lat, wk, wv, block_ids, n_blocks, num_blocks, per_wg, ex);
  else
    expand_blocks<64><<<grid, (64 + kDV) / 32 * 64, 0, s>>>(p, lat, wk, wv, block_ids, n_blocks, num_blocks, per_wg, ex);
  return hipGetLastError();
}

}  // namespace gqla
