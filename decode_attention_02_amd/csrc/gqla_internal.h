// Internal declarations shared by the host API and the HIP kernels of libgqla.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

struct gqla_dims;   // include/gqla.h

namespace gqla {

// Message returned by gqla_last_error() on the calling thread (gqla_api.cpp).
void set_last_error(const char* msg);

constexpr int kBlock = 64;        // tokens per cache block
constexpr int kSlab = 32;         // key features per slab of the expanded cache
constexpr int kHalf = 32;         // tokens per value half-slab of the expanded cache
constexpr int kNumCUs = 256;      // MI355X compute units (split-KV planning)

enum OutKind : int32_t { OUT_F32 = 0, OUT_BF16 = 1 };

// One split-KV attention launch. A "kv head" is the latent (absorb path, 1 per
// sequence) or one group's expanded K/V (GQA path, G per sequence). Row r of a kv head
// is query row i = r / heads_per_kv of head h = kvh * heads_per_kv + r % heads_per_kv.
struct AttnParams {
  const void* q;                 // [B][s_q][H][dk] data
  const void* kv;                // cache pool base (data)
  const int32_t* block_table;    // [B][max_blocks]
  const int32_t* ctx_lens;       // [B]
  int64_t num_blocks;
  int64_t block_stride;          // elements per physical block
  int64_t kvh_stride;            // elements between kv heads inside a block
  int32_t max_blocks;
  int32_t B, H, s_q;
  int32_t kv_heads, heads_per_kv;
  int32_t dk, dvo;               // key width, value/output width
  int32_t k_ts, k_fs;            // K(t, f) at k_ts * t + k_fs * f (k_slab == 0)
  int32_t k_slab;                // > 0: K in feature slabs of this width (see kv_k_index)
  int32_t k_own;                 // with a shared RoPE key: K features [0, k_own) in the group
                                 // chunk, the rest in the block's shared key area (else = dk)
  int64_t kv_off;                // elements from a block's start to its group 0 chunk
  int32_t v_off, v_half, v_ts, v_fs;   // V(t, f) at v_off + v_half*(t/32) + v_ts*(t%32) + v_fs*f
  float scale;
  int32_t n_split, blocks_per_split;
  // Length-balanced plan (GQA path, chunks > 0): the batch's blocks, laid end to end in
  // sequence order, are cut into `chunks` equal runs of at least `chunk_min` blocks per
  // group; a run may end one sequence and start the next. n_split is then the number of
  // partial slots per row and `decl_blocks` the blocks of the declared longest context.
  int32_t chunks, chunk_min, decl_blocks;
  float* ws_o;                   // [B*s_q*H][n_split][dvo]   (n_split > 1)
  float* ws_lse;                 // [B*s_q*H][n_split]        (n_split > 1)
  void* out;                     // [B*s_q*H][dvo]            (n_split == 1)
  int32_t out_kind;              // OutKind of `out`
  float* lse;                    // [B*s_q*H] or null         (n_split == 1)
};

struct CombineParams {
  const float* ws_o;
  const float* ws_lse;
  int32_t rows, n_split, dvo;
  void* out;
  int32_t out_kind;
  float* lse;
};

struct ProjParams {
  int32_t rows;                  // B * s_q
  int32_t H, G, dc, dr, dn, dv;
  int32_t rope_shared;           // expanded layout: RoPE key once per block
};

// Generic kernels: any dims that fit the LDS budget, fp32 or bf16 data.
hipError_t launch_generic_attn(const AttnParams& p, bool bf16, hipStream_t s);
size_t generic_attn_lds_bytes(int dk, int dvo);
hipError_t launch_combine(const CombineParams& c, hipStream_t s);
hipError_t launch_generic_absorb_query(const ProjParams& d, const void* q_nope, const void* q_rope,
                                       const void* w_uk, void* q_abs, bool bf16, hipStream_t s);
hipError_t launch_generic_out_proj(const ProjParams& d, const float* o_lat, const void* w_uv,
                                   void* out, bool bf16, hipStream_t s);
// Output side: y[M][N] = x[M][K] w[N][K]^T (x fp32 or the data type), and the fold of
// W_UV^g into W_O.
hipError_t launch_out_hidden(const void* x, bool x_f32, const void* w, void* y, int M, int N, int K, bool bf16,
                             hipStream_t s);
hipError_t launch_fold_out_weight(const ProjParams& p, int hidden, const void* w_o, const void* w_uv, void* w_fold,
                                  bool bf16, hipStream_t s);
// Element offsets inside one block of the expanded cache (both layouts; see gqla.h).
struct ExpandedLayout {
  int64_t block;      // elements per block
  int64_t rope;       // elements of the shared RoPE key area at the block's start (0 if none)
  int64_t chunk;      // elements per group chunk
  int32_t k_feats;    // K features stored in each group chunk (d_qk, or d_n when shared)
};
__host__ __device__ inline ExpandedLayout expanded_layout(int dn, int dr, int dv, int G, bool shared) {
  ExpandedLayout l;
  l.k_feats = shared ? dn : dn + dr;
  l.rope = shared ? static_cast<int64_t>(kBlock) * dr : 0;
  l.chunk = static_cast<int64_t>(kBlock) * (l.k_feats + dv);
  l.block = l.rope + l.chunk * G;
  return l;
}

hipError_t launch_generic_expand(const ProjParams& d, const void* latent, const void* w_uk,
                                 const void* w_uv, const int32_t* block_ids, int64_t n_blocks,
                                 int64_t num_blocks, void* expanded, bool bf16, hipStream_t s);

// One append call: the s_q new tokens of every sequence (n_tok = B * s_q).
struct AppendParams {
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int32_t max_blocks;
  int64_t num_blocks;
  int32_t n_tok, s_q, G;
  int32_t dc, dr, dn, dv;
  int32_t rope_shared;
  float rope_theta;
  double inv_freq[64];   // rope_theta^(-2k/d_R), k < d_R / 2 (fp64, from the host)
};
hipError_t launch_append(const AppendParams& a, const void* c_new, const void* kr_new, const void* w_uk,
                         const void* w_uv, void* latent, void* expanded, bool bf16, hipStream_t s);

// Decode-step estimate of each path (microseconds) on MI355X; path_model.cpp.
struct PathEstimate {
  double absorb_us, gqa_us;
};
PathEstimate estimate_paths(const ::gqla_dims* d, int64_t total_ctx, int n_split_abs, int n_split_gqa);

}  // namespace gqla
