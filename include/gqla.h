/*
 * gqla.h — C ABI of libgqla.so: the decode-attention hot path of Group-Query Latent
 * Attention (GQLA) on AMD Instinct MI355X (gfx950).
 *
 * GQLA caches MLA's joint low-rank latent c_KV per token and gives each group of
 * gs = H / G query heads one shared key up-projection W_UK^g and one shared value
 * up-projection W_UV^g ("GQLA: Group-Query Latent Attention for Hardware-Adaptive
 * Decoding", Abstract). The same weights decode two algebraically equivalent ways
 * ("GQLA: Attention latente par requêtes groupées ...", English abstract):
 *
 *   (a) MQA-absorb: gqla_absorb_query -> gqla_decode_absorb -> gqla_out_proj.
 *       W_UK^g is folded into every query, all heads attend over the cached latent,
 *       and W_UV^g is applied to each head's latent output.
 *   (b) GQA: gqla_expand_cache (when latent blocks are filled) -> gqla_decode_gqa.
 *       The latent is expanded into G key/value heads that the gs query heads of each
 *       group share ("Grouped Query Attention (GQA)", section "Fonctionnement de la GQA").
 *
 * Conventions shared by every call
 * --------------------------------
 * Dimensions: B batch, H query heads, G groups (G divides H; head h is in group
 * h / gs), d_c latent rank, d_R RoPE dim, d_n nope dim, d_qk = d_n + d_R, d_v value
 * dim, s_q >= 1 query rows per sequence (1 for plain decode; 2 or more when a multi-token
 * prediction head proposes tokens that are verified together, as the pages run the GQA path
 * at s_q = 2). Any s_q is accepted; shapes the MFMA kernels do not cover (absorb path:
 * H * s_q not in {16, 32, ..., 512}; GQA path: gs * s_q > 32) run on the generic kernels.
 *
 * Element type: every tensor marked "data" is float (GQLA_F32) or bfloat16 (GQLA_BF16)
 * as dims->dtype says; accumulation is always fp32. o_lat, lse and the workspace are
 * always fp32. Index tensors are int32.
 *
 * Memory: every pointer except dims/paged and the `bytes`/`n` out-parameters is DEVICE
 * memory owned by the caller, contiguous in the layout stated. The library allocates
 * nothing, keeps no state between calls beyond a thread-local error string, and never
 * synchronises: work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 * Calls may be captured in a HIP graph (no memset nodes are recorded).
 *
 * Paged caches: tokens live in fixed 64-token blocks ("Grouped Query Attention (GQA)",
 * section "GQA et techniques connexes", PagedAttention). Logical token t of sequence b
 * is slot t % 64 of physical block block_table[b][t / 64].
 *
 * Causality: ctx_lens[b] = L_b counts the s_q new tokens. Query row i (0 <= i < s_q)
 * of sequence b sees tokens 0 .. L_b - s_q + i.
 *
 * Softmax scale: dims->softmax_scale, or 1/sqrt(d_n + d_R) when it is <= 0; the same
 * value must be used on both paths for them to agree.
 *
 * Errors: calls return a gqla_status and never abort. Host-visible argument problems
 * (null pointer, H % G != 0, s_q < 1, block_size != 64, non-positive dims, unknown
 * dtype or path, workspace too small, dims the kernels do not cover) are reported
 * before anything is launched. Device-side metadata is guarded inside the kernels:
 * a block id outside [0, num_blocks) is never dereferenced, and every output row that
 * would have read it, or that sees no token (L_b < s_q), or whose L_b exceeds
 * max_blocks_per_seq * 64 is written as NaN. gqla_last_error() gives a message for the
 * most recent failing call on the calling thread.
 */
#ifndef GQLA_H
#define GQLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqla_status {
  GQLA_OK = 0,
  GQLA_ERR_INVALID_ARG = -1,  /* bad argument; nothing launched */
  GQLA_ERR_UNSUPPORTED = -2,  /* valid dims that no kernel covers; nothing launched */
  GQLA_ERR_WORKSPACE = -3,    /* workspace smaller than gqla_workspace_bytes() */
  GQLA_ERR_HIP = -4           /* a HIP launch or runtime call failed */
} gqla_status;

typedef enum gqla_dtype { GQLA_F32 = 0, GQLA_BF16 = 1 } gqla_dtype;

typedef enum gqla_path { GQLA_PATH_ABSORB = 0, GQLA_PATH_GQA = 1 } gqla_path;

/* Shape of one GQLA attention layer at decode time. */
typedef struct gqla_dims {
  int32_t batch;        /* B   >= 1 */
  int32_t num_heads;    /* H   >= 1 */
  int32_t num_groups;   /* G   >= 1, divides H */
  int32_t latent_rank;  /* d_c >= 1 */
  int32_t rope_dim;     /* d_R >= 0 */
  int32_t nope_dim;     /* d_n >= 1 */
  int32_t v_dim;        /* d_v >= 1 */
  int32_t s_q;          /* >= 1 query rows per sequence */
  int32_t block_size;   /* tokens per cache block; must be 64 */
  int32_t dtype;        /* gqla_dtype of every "data" tensor */
  float softmax_scale;  /* <= 0 selects 1/sqrt(d_n + d_R) */
  int32_t rope_shared;  /* expanded-cache layout (GQA path): 0 = the RoPE key in every
                           group's K; 1 = stored once per block and shared by the groups
                           (see gqla_expand_cache) */
} gqla_dims;

/* Paged-cache metadata for one decode batch. */
typedef struct gqla_paged {
  const int32_t* block_table; /* device int32 [B][max_blocks_per_seq]; entries past a
                                 sequence's last block are never read */
  const int32_t* ctx_lens;    /* device int32 [B]; L_b, includes the s_q new tokens */
  int32_t max_blocks_per_seq; /* row length of block_table, >= 1 */
  int32_t max_ctx_len;        /* host-known upper bound on every L_b, >= s_q; sizes the
                                 split-KV plan and must not be exceeded */
  int64_t num_blocks;         /* physical blocks in the cache pool, >= 1 */
  int32_t num_splits;         /* 0: automatic split-KV plan; k > 0: k splits */
} gqla_paged;

/*
 * gqla_absorb_query — fold W_UK^g into the queries (MQA-absorb path, step 1).
 *   q_abs[b][i][h] = [ W_UK^g^T q_nope[b][i][h] ; q_rope[b][i][h] ],  g = h / gs.
 * ("GQLA: Attention latente ...", English abstract: the MQA-absorb path is MLA's
 * absorbed form; gqla_attn.py docstring: the up-projection is absorbed into the query.)
 *   q_nope : data [B][s_q][H][d_n]
 *   q_rope : data [B][s_q][H][d_R]   (already rotated to the row's position)
 *   w_uk   : data [G][d_n][d_c]      (out x in, like a linear layer's weight)
 *   q_abs  : data [B][s_q][H][d_c + d_R]   (output, rounded to the data type)
 */
gqla_status gqla_absorb_query(const gqla_dims* dims, const void* q_nope, const void* q_rope,
                              const void* w_uk, void* q_abs, void* stream);

/*
 * gqla_decode_absorb — every head attends over the shared latent "key head" (step 2).
 *   s_t = scale * <q_abs[b][i][h], [c_t | kr_t]>,  o_lat = sum_t softmax(s)_t c_t,
 * over the visible tokens t of row i; split-KV with an online-softmax merge.
 * ("GQLA: Attention latente ...", English abstract: the MQA-absorb path keeps MLA's absorbed
 * form, in which all query heads share one latent key/value head; gqla_attn.py docstring:
 * the absorbed path attends with a single MQA-style head per layer.)
 *   q_abs        : data [B][s_q][H][d_c + d_R]
 *   latent_cache : data [num_blocks][64][d_c + d_R]; row = [c_KV (d_c) | k_rope (d_R)]
 *   workspace    : fp32 scratch of at least gqla_workspace_bytes(.., GQLA_PATH_ABSORB)
 *                  bytes (may be NULL when that is 0)
 *   o_lat        : fp32 [B][s_q][H][d_c]  (output)
 *   lse          : fp32 [B][s_q][H] log-sum-exp of the scaled scores (output; NULL = skip)
 */
gqla_status gqla_decode_absorb(const gqla_dims* dims, const gqla_paged* paged,
                               const void* q_abs, const void* latent_cache, void* workspace,
                               size_t workspace_bytes, float* o_lat, float* lse, void* stream);

/*
 * gqla_decode_absorb_noalloc — gqla_decode_absorb without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The split-KV partial results go to a fixed scratch array
 * of GQLA_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per GPU, held from
 * the library's load until the process ends; the call itself allocates nothing.
 *   Arguments and results are those of gqla_decode_absorb (same kernels, same outputs).
 *   The scratch of the calling thread's current device is used: `stream` must belong to it.
 *   Its address is looked up on the first call on each device; make that first call outside
 *   graph capture.
 *   Calls that overlap on one GPU (on different streams, or from several threads) share the
 *   array and race: serialise them. Nothing in it needs clearing between calls.
 * Errors: those of gqla_decode_absorb, and GQLA_ERR_WORKSPACE when the split plan needs more
 * than GQLA_NOALLOC_SCRATCH_BYTES (B * s_q * H * n_split * (d_c + 1) * 4 bytes; e.g. LLaMA-3-8B
 * batch 32 at s_q = 1 needs 16.8 MB, the DeepSeek-V3 long-context batch of 8 at s_q = 2 needs
 * 33.6 MB; see gqla_workspace_bytes).
 */
#define GQLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gqla_status gqla_decode_absorb_noalloc(const gqla_dims* dims, const gqla_paged* paged, const void* q_abs,
                                       const void* latent_cache, float* o_lat, float* lse, void* stream);

/*
 * gqla_out_proj — apply W_UV^g to each head's latent output (step 3).
 *   out[b][i][h] = W_UV^g o_lat[b][i][h],  g = h / gs.
 * (The value up-projection is shared by the group ("GQLA: Group-Query Latent Attention for
 * Hardware-Adaptive Decoding", Abstract: group-shared up-projections), and applying it
 * after the attention average instead of to every cached token gives the same result by
 * linearity, which is what makes the absorbed form equivalent ("GQLA: Attention latente
 * ...", English abstract; gqla_attn.py docstring, MQA-absorb path).)
 *   o_lat : fp32 [B][s_q][H][d_c];  w_uv : data [G][d_v][d_c];  out : data [B][s_q][H][d_v]
 */
gqla_status gqla_out_proj(const gqla_dims* dims, const float* o_lat, const void* w_uv,
                          void* out, void* stream);

/*
 * gqla_decode_absorb_out — gqla_decode_absorb followed by gqla_out_proj, in one call (steps 2
 * and 3 of the MQA-absorb path). When the decode is split, the split combine and the W_UV^g
 * product run as one kernel that keeps the merged latent rows on chip; unsplit, or at shapes
 * without that kernel, it is exactly the two calls.
 *   q_abs, latent_cache, workspace, lse : as gqla_decode_absorb (same workspace size)
 *   w_uv  : data [G][d_v][d_c]
 *   o_lat : fp32 [B][s_q][H][d_c]  (output; the latent rows are written on every form)
 *   out   : data [B][s_q][H][d_v]  (output)
 * Errors: those of gqla_decode_absorb and gqla_out_proj.
 */
gqla_status gqla_decode_absorb_out(const gqla_dims* dims, const gqla_paged* paged, const void* q_abs,
                                   const void* latent_cache, const void* w_uv, void* workspace,
                                   size_t workspace_bytes, float* o_lat, void* out, float* lse, void* stream);

/*
 * gqla_expand_cache — expand latent blocks into the per-group K/V cache (GQA path).
 * For each listed block p, group g and slot r (gqla_attn.py docstring: the latent is
 * expanded into num_groups full key/value heads):
 *   K[p][g][r] = [ W_UK^g c_r ; kr_r ]   (d_qk values; the RoPE key is copied per group)
 *   V[p][g][r] =   W_UV^g c_r            (d_v values)
 *   latent_cache   : data [num_blocks][64][d_c + d_R]
 *   w_uk, w_uv     : data [G][d_n][d_c], [G][d_v][d_c]
 *   block_ids      : device int32 [n_blocks], physical blocks to (re)expand; ids outside
 *                    [0, num_blocks) are skipped
 *   expanded_cache : rope_shared = 0: data [num_blocks][G][64*d_qk + d_v*64]; per (block,
 *                    group) chunk: K = [k_nope | k_rope] in slabs of 32 features: slab s
 *                    holds features [32s, 32s + w_s), w_s = min(32, d_qk - 32s), for all
 *                    64 slots, slot-major (feature f of slot r at 2048*(f/32) + r*w_s +
 *                    f%32); then V in two halves of 32 slots, each feature-major [d_v][32]
 *                    (feature f of slot r at 64*d_qk + 32*d_v*(r/32) + 32*f + r%32).
 *                    rope_shared = 1: per block, first the RoPE keys of its 64 slots once
 *                    ([64*d_R], slabs of 32 as above over the d_R features), then per
 *                    group a chunk of 64*d_n + d_v*64: k_nope in slabs over the d_n
 *                    features, then V as above (64*d_n in place of 64*d_qk); a block is
 *                    64*d_R + G*64*(d_n + d_v) values (gqla_cache_bytes_per_token * 64).
 *                    (With these slabs each wide load of the decode kernel covers
 *                    whole 128-byte lines of a bf16 cache.)
 */
gqla_status gqla_expand_cache(const gqla_dims* dims, const void* latent_cache, const void* w_uk,
                              const void* w_uv, const int32_t* block_ids, int64_t n_blocks,
                              int64_t num_blocks, void* expanded_cache, void* stream);

/*
 * gqla_decode_gqa — grouped-query decode over the expanded cache.
 *   out[b][i][h] = sum_t softmax(scale * <q[b][i][h], K[g]_t>)_t V[g]_t,  g = h / gs,
 * over the visible tokens t of row i; split-KV with an online-softmax merge. With
 * num_splits = 0, when the (sequence, group) pairs cannot cover the 256 CUs and the context
 * has to be split (batch <= 256), the batch's blocks are cut into equal runs per group on
 * the device, from ctx_lens (the length-balanced plan of gqla_num_splits).
 * (The gs query heads of a group share one key head and one value head: "Grouped Query
 * Attention (GQA)", section "Fonctionnement de la GQA"; GQLA's GQA path runs that over the
 * latent expanded into G key/value heads: gqla_attn.py docstring, and "GQLA: Attention
 * latente ...", English abstract, where it is the path for low-compute GPUs at s_q = 2.)
 *   q              : data [B][s_q][H][d_qk] = [q_nope | q_rope]
 *   expanded_cache : layout of gqla_expand_cache
 *   workspace      : fp32 scratch of at least gqla_workspace_bytes(.., GQLA_PATH_GQA)
 *   out            : data [B][s_q][H][d_v]  (output)
 *   lse            : fp32 [B][s_q][H] (output; NULL = skip)
 */
gqla_status gqla_decode_gqa(const gqla_dims* dims, const gqla_paged* paged, const void* q,
                            const void* expanded_cache, void* workspace, size_t workspace_bytes,
                            void* out, float* lse, void* stream);

/*
 * gqla_append_tokens — write each sequence's s_q new tokens into the paged caches (the
 * step before decode: the latent comes out of the down-projection and, on the GQA path,
 * is expanded into the groups' K/V — "GQLA: Attention latente ...", English abstract;
 * gqla_attn.py docstring). For row i of sequence b, at position t = L_b - s_q + i:
 *   latent_cache[block_table[b][t / 64]][t % 64] = [ c_new[b][i] ; RoPE_t(kr_new[b][i]) ]
 * and, when expanded_cache is not NULL, that slot's K and V for every group, as
 * gqla_expand_cache would write them from the new latent row. RoPE pairs component k with
 * k + d_R/2 and rotates the pair by t * rope_theta^(-2k/d_R) (computed in fp64, rounded
 * once to the data type); the pages do not describe RoPE, this is the half-split form.
 *   c_new          : data [B][s_q][d_c]
 *   kr_new         : data [B][s_q][d_R], not yet rotated (may be NULL when d_R = 0)
 *   rope_theta     : > 0 (10000 for the workloads here)
 *   w_uk, w_uv     : data [G][d_n][d_c], [G][d_v][d_c] (needed only with expanded_cache)
 *   latent_cache   : data [num_blocks][64][d_c + d_R] (updated in place), or NULL for a
 *                    GQA-only deployment that keeps only the expanded cache
 *   expanded_cache : layout of gqla_expand_cache, or NULL for an absorb-only deployment
 *                    (at least one of the two caches must be given)
 * Sequences with s_q > L_b or L_b beyond the table, and tokens whose block id lies outside
 * [0, num_blocks), are skipped (nothing written). Requires d_R even, d_c % 8 == 0 and
 * 64 * (d_c + d_R) <= 160 KiB; errors: GQLA_ERR_INVALID_ARG / GQLA_ERR_UNSUPPORTED.
 */
gqla_status gqla_append_tokens(const gqla_dims* dims, const gqla_paged* paged, const void* c_new,
                               const void* kr_new, float rope_theta, const void* w_uk, const void* w_uv,
                               void* latent_cache, void* expanded_cache, void* stream);

/*
 * Output side: the layer's output projection W_O after the heads (gqla_attn.py module
 * source, GQLAAttention: a bias-free out_proj from H*head_dim to hidden_size applied to
 * the heads' outputs laid side by side head-major), on either path.
 *
 * gqla_out_hidden — y = x W^T over the B*s_q rows of the batch:
 *   folded = 0: x = the heads' outputs, data [B][s_q][H][d_v] (gqla_out_proj or
 *               gqla_decode_gqa output), w = W_O, data [hidden][H*d_v]:
 *               y[r][n] = sum_{h,v} W_O[n][h*d_v + v] x[r][h][v];
 *   folded = 1: x = the absorb path's latent outputs, fp32 [B][s_q][H][d_c]
 *               (gqla_decode_absorb output, no gqla_out_proj), w = W_fold from
 *               gqla_fold_out_weight, data [hidden][H*d_c]:
 *               y[r][n] = sum_{h,c} W_fold[n][h*d_c + c] x[r][h][c];
 *   y : data [B][s_q][hidden] (output; fp32 accumulation, rounded once to the data type).
 * Both give the same y up to rounding. hidden is free (the configurations fix none; the
 * module ties it to H * head_dim). The fold reads d_c / d_v times more weight bytes per
 * step than W_O plus W_UV, so at decode batch sizes it is the slower form on MI355X.
 * Errors: GQLA_ERR_INVALID_ARG for bad dims, hidden outside [1, 65535] or NULL pointers.
 */
gqla_status gqla_out_hidden(const gqla_dims* dims, int32_t hidden, int32_t folded, const void* x,
                            const void* w, void* y, void* stream);

/*
 * gqla_fold_out_weight — W_O with every head's W_UV^g folded in (once per model):
 *   W_fold[n][h*d_c + c] = sum_v W_O[n][h*d_v + v] W_UV^g[v][c],  g = h / gs.
 *   w_o : data [hidden][H*d_v];  w_uv : data [G][d_v][d_c];  w_fold : data [hidden][H*d_c]
 * (fp32 accumulation, rounded once to the data type). Errors as gqla_out_hidden.
 */
gqla_status gqla_fold_out_weight(const gqla_dims* dims, int32_t hidden, const void* w_o, const void* w_uv,
                                 void* w_fold, void* stream);

/* Number of partial results per query row the decode call for `path` will form (host
 * arithmetic only): its KV splits, or, for the GQA path's length-balanced plan (chosen when
 * num_splits is 0, batch x groups < 256 CUs and the context is split), an upper bound on the
 * equal block runs one sequence can meet, min(ceil(256 / G) + 1, ceil(max blocks / 8) + 1). */
gqla_status gqla_num_splits(const gqla_dims* dims, const gqla_paged* paged, int32_t path,
                            int32_t* n);

/* Workspace bytes the decode call for `path` needs (0 when it runs unsplit). */
gqla_status gqla_workspace_bytes(const gqla_dims* dims, const gqla_paged* paged, int32_t path,
                                 size_t* bytes);

/*
 * gqla_pick_path — which decode path to run for a batch on MI355X (host arithmetic only).
 * The two paths compute the same attention ("GQLA: Attention latente ...", English abstract:
 * GQLA decodes either as MQA-absorb or as GQA; gqla_attn.py's decode_path switch), but trade
 * cache traffic for computation, so the faster one depends on the hardware. This returns
 * the path whose estimated decode step (absorbed query + latent decode + value projection,
 * against expansion of the new tokens' blocks + grouped decode, each with its split
 * combine) is shorter, from the per-step bytes and flops of these kernels and throughputs
 * measured for them on MI355X. Ties go to the absorb path (the smaller cache).
 *   total_ctx : sum of the batch's context lengths (each includes its s_q new tokens)
 *   max_ctx   : longest context in the batch
 *   path      : (output) GQLA_PATH_ABSORB or GQLA_PATH_GQA
 *   est_us    : (output, NULL = skip) float[2]: estimated step microseconds {absorb, gqa}
 * Errors: GQLA_ERR_INVALID_ARG for bad dims or total_ctx outside [B * s_q, B * max_ctx].
 * The GQA path also needs the expanded cache, G * (d_qk + d_v) values per token: the
 * caller decides whether that fits (gqla_cache_bytes_per_token).
 */
gqla_status gqla_pick_path(const gqla_dims* dims, int64_t total_ctx, int32_t max_ctx, int32_t* path,
                           float* est_us);

/* Cache bytes per token per layer: latent (d_c + d_R) * elt for the absorb path,
 * G * (d_qk + d_v) * elt for the GQA path (G * (d_n + d_v) * elt + d_R * elt with
 * rope_shared); 0 for invalid arguments. For LLaMA-3-8B converted to GQLA the latent is
 * 576 values against the 8-KV-head GQA baseline's 2048, 28.125% ("GQLA: Attention latente
 * ...", English abstract); a GQA cache of 8 KV heads of 128 values is 2 * 8 * 128 * 2 B =
 * 4 KiB per token per layer, 128 KiB over 32 layers ("Grouped Query Attention (GQA)",
 * section "Pourquoi la GQA réduit le cache KV"). */
int64_t gqla_cache_bytes_per_token(const gqla_dims* dims, int32_t path);

/* Synchronous debug check of device-side paged metadata: copies block_table and ctx_lens
 * to the host and verifies s_q <= L_b <= min(max_ctx_len, 64 * max_blocks_per_seq) and
 * 0 <= id < num_blocks for every block a sequence uses. Returns GQLA_ERR_INVALID_ARG with
 * the first offending (b, block) in gqla_last_error(). */
gqla_status gqla_validate_paged(const gqla_dims* dims, const gqla_paged* paged, void* stream);

/*
 * gqla_stream_read — measurement helper, not a decode step: reads `bytes` bytes at `src`
 * (device memory, 16-byte aligned, bytes a non-zero multiple of 16) with the load form the
 * decodes stream their caches with (non-temporal 128-bit loads covering whole lines), over
 * num_wgs workgroups of 256 lanes in [1, 65536], and writes each workgroup's fp32 sum of the
 * data read as fp32 words to partial[num_wgs] (device, caller-owned), so the loads cannot be
 * dropped. Timing it gives the streaming-read rate the decodes' HBM fraction is set beside.
 * Errors: GQLA_ERR_INVALID_ARG for NULL pointers, a misaligned src or size, or num_wgs out of
 * range; GQLA_ERR_HIP if the launch fails.
 */
gqla_status gqla_stream_read(const void* src, size_t bytes, float* partial, int32_t num_wgs, void* stream);

const char* gqla_status_string(gqla_status status);
const char* gqla_last_error(void);

/* Library version string. */
const char* gqla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQLA_H */
