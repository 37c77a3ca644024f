// Host side of libgqla: argument validation, split-KV planning and kernel dispatch.
// Nothing here allocates device memory or synchronises (except gqla_validate_paged,
// a debug call documented as synchronous).
#include "../../include/gqla.h"
#include "gqla_internal.h"
#include "tuned.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

gqla_status fail(gqla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

void gqla::set_last_error(const char* msg) { g_err = msg; }

namespace {

gqla_status hip_fail(hipError_t e, const char* where) {
  return fail(GQLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

gqla_status check_dims(const gqla_dims* d) {
  if (d == nullptr) return fail(GQLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->num_heads < 1 || d->num_groups < 1 || d->latent_rank < 1 ||
      d->rope_dim < 0 || d->nope_dim < 1 || d->v_dim < 1)
    return fail(GQLA_ERR_INVALID_ARG, "dimensions must be positive (rope_dim >= 0)");
  if (d->num_heads % d->num_groups != 0)
    return fail(GQLA_ERR_INVALID_ARG, "num_groups (%d) must divide num_heads (%d)", d->num_groups, d->num_heads);
  if (d->s_q < 1) return fail(GQLA_ERR_INVALID_ARG, "s_q must be >= 1 (got %d)", d->s_q);
  if (d->block_size != gqla::kBlock)
    return fail(GQLA_ERR_INVALID_ARG, "block_size must be 64 (got %d)", d->block_size);
  if (d->dtype != GQLA_F32 && d->dtype != GQLA_BF16)
    return fail(GQLA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->rope_shared != 0 && d->rope_shared != 1)
    return fail(GQLA_ERR_INVALID_ARG, "rope_shared must be 0 or 1 (got %d)", d->rope_shared);
  return GQLA_OK;
}

gqla_status check_path(int32_t path) {
  if (path != GQLA_PATH_ABSORB && path != GQLA_PATH_GQA)
    return fail(GQLA_ERR_INVALID_ARG, "unknown path %d (0 = absorb, 1 = gqa)", path);
  return GQLA_OK;
}

gqla_status check_paged(const gqla_dims* d, const gqla_paged* p) {
  if (p == nullptr) return fail(GQLA_ERR_INVALID_ARG, "paged is NULL");
  if (p->block_table == nullptr || p->ctx_lens == nullptr)
    return fail(GQLA_ERR_INVALID_ARG, "block_table and ctx_lens must be device pointers");
  if (p->max_blocks_per_seq < 1 || p->num_blocks < 1)
    return fail(GQLA_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be >= 1");
  if (p->max_ctx_len < d->s_q)
    return fail(GQLA_ERR_INVALID_ARG, "max_ctx_len (%d) must be >= s_q (%d)", p->max_ctx_len, d->s_q);
  if (static_cast<int64_t>(p->max_ctx_len) > static_cast<int64_t>(p->max_blocks_per_seq) * gqla::kBlock)
    return fail(GQLA_ERR_INVALID_ARG, "max_ctx_len (%d) exceeds max_blocks_per_seq * 64", p->max_ctx_len);
  if (p->num_splits < 0) return fail(GQLA_ERR_INVALID_ARG, "num_splits must be >= 0");
  return GQLA_OK;
}

float resolve_scale(const gqla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale
                                : 1.0f / std::sqrt(static_cast<float>(d->nope_dim + d->rope_dim));
}

int elt_bytes(const gqla_dims* d) { return d->dtype == GQLA_BF16 ? 2 : 4; }

int nblk_declared(const gqla_paged* p) { return p->max_ctx_len / gqla::kBlock + (p->max_ctx_len % gqla::kBlock != 0); }

struct Plan {
  int n_split;
  int blocks_per_split;
  bool tuned;
  int chunks = 0;      // > 0: length-balanced GQA plan (see below)
  int chunk_min = 0;
};

// Split-KV plan. Units of independent work are (sequence, group) on the GQA path and
// sequences on the absorb path; the context is cut into equal 64-token-aligned splits
// until the launch holds enough workgroups to cover the 256 CUs, while keeping each
// split long enough to amortise its prologue and the partial-result traffic.
Plan plan(const gqla_dims* d, const gqla_paged* p, int32_t path) {
  Plan pl{};
  const int nblk = nblk_declared(p);
  int n;
  if (path == GQLA_PATH_GQA) {
    pl.tuned = gqla::tuned_gqa_supported(d);
    const int64_t units = static_cast<int64_t>(d->batch) * d->num_groups;
    const int64_t target = pl.tuned ? gqla::tuned_gqa_target_wgs() : 2 * gqla::kNumCUs;
    const int min_blocks = pl.tuned ? gqla::tuned_gqa_min_blocks_per_split() : 2;
    n = static_cast<int>(std::min<int64_t>((target + units - 1) / units, std::max(1, nblk / min_blocks)));
  } else {
    pl.tuned = gqla::tuned_absorb_supported(d);
    const int64_t units = pl.tuned ? d->batch
                                   : static_cast<int64_t>(d->batch) * ((d->num_heads * d->s_q + 15) / 16);
    const int64_t target = pl.tuned ? gqla::tuned_absorb_target_wgs(d) : 2 * gqla::kNumCUs;
    const int min_blocks = pl.tuned ? gqla::tuned_absorb_min_blocks_per_split() : 2;
    n = static_cast<int>(std::min<int64_t>((target + units - 1) / units, std::max(1, nblk / min_blocks)));
  }
  if (p->num_splits > 0) n = p->num_splits;
  n = std::max(1, std::min(n, std::min(nblk, 1024)));
  if (path == GQLA_PATH_ABSORB && pl.tuned)   // the kernel stages one split's block ids in LDS
    n = std::max(n, (nblk + gqla::tuned_absorb_max_blocks_per_split() - 1) / gqla::tuned_absorb_max_blocks_per_split());
  pl.blocks_per_split = (nblk + n - 1) / n;
  pl.n_split = (nblk + pl.blocks_per_split - 1) / pl.blocks_per_split;
  // When the context must be split to cover the CUs and the split count is left to the
  // plan, the tuned GQA kernel cuts the batch's blocks (sequences laid end to end) into
  // equal runs per group instead: with ragged lengths, equal splits of each sequence give
  // the workgroups of the longest one the most blocks while those of the shortest idle.
  // A sequence of n blocks meets at most ceil(n / run) + 1 runs, which bounds the partial
  // slots per row; the kernel marks the slots a sequence does not use as empty.
  if (path == GQLA_PATH_GQA && pl.tuned && p->num_splits == 0 && pl.n_split > 1 && d->batch <= gqla::kNumCUs &&
      static_cast<int64_t>(d->batch) * nblk < (int64_t{1} << 30)) {
    pl.chunks = static_cast<int>((gqla::tuned_gqa_target_wgs() + d->num_groups - 1) / d->num_groups);
    pl.chunk_min = gqla::tuned_gqa_min_blocks_per_split();
    pl.n_split = std::min(pl.chunks + 1, (nblk + pl.chunk_min - 1) / pl.chunk_min + 1);
    pl.blocks_per_split = nblk;
  }
  return pl;
}

size_t workspace_for(const gqla_dims* d, int32_t path, int n_split) {
  if (n_split <= 1) return 0;
  const size_t rows = static_cast<size_t>(d->batch) * d->s_q * d->num_heads;
  const size_t dvo = path == GQLA_PATH_GQA ? d->v_dim : d->latent_rank;
  return rows * n_split * (dvo + 1) * sizeof(float);
}

// The split-KV decode of either path; with skip_combine the partials are left in the
// workspace for a fused consumer (gqla_decode_absorb_out).
gqla_status run_decode(const gqla_dims* d, const gqla_paged* pg, int32_t path, const void* q,
                       const void* cache, void* ws, size_t ws_bytes, void* out, int32_t out_kind,
                       float* lse, void* stream, bool skip_combine = false) {
  const Plan pl = plan(d, pg, path);
  const size_t need = workspace_for(d, path, pl.n_split);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(GQLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  const bool gqa = path == GQLA_PATH_GQA;
  gqla::AttnParams a{};
  a.q = q;
  a.kv = cache;
  a.block_table = pg->block_table;
  a.ctx_lens = pg->ctx_lens;
  a.num_blocks = pg->num_blocks;
  a.max_blocks = pg->max_blocks_per_seq;
  a.B = d->batch;
  a.H = d->num_heads;
  a.s_q = d->s_q;
  a.scale = resolve_scale(d);
  a.n_split = pl.n_split;
  a.blocks_per_split = pl.blocks_per_split;
  a.chunks = pl.chunks;
  a.chunk_min = pl.chunk_min;
  a.decl_blocks = nblk_declared(pg);
  const int rows = d->batch * d->s_q * d->num_heads;
  if (gqa) {
    const int dqk = d->nope_dim + d->rope_dim;
    a.kv_heads = d->num_groups;
    a.heads_per_kv = d->num_heads / d->num_groups;
    a.dk = dqk;
    a.dvo = d->v_dim;
    const gqla::ExpandedLayout lay =
        gqla::expanded_layout(d->nope_dim, d->rope_dim, d->v_dim, d->num_groups, d->rope_shared != 0);
    a.kvh_stride = lay.chunk;
    a.block_stride = lay.block;
    a.kv_off = lay.rope;
    a.k_own = lay.k_feats;
    a.k_ts = 0;
    a.k_fs = 0;
    a.k_slab = gqla::kSlab;
    a.v_off = gqla::kBlock * lay.k_feats;
    a.v_half = gqla::kHalf * d->v_dim;
    a.v_ts = 1;
    a.v_fs = gqla::kHalf;
  } else {
    const int dq = d->latent_rank + d->rope_dim;
    a.kv_heads = 1;
    a.heads_per_kv = d->num_heads;
    a.dk = dq;
    a.dvo = d->latent_rank;
    a.kvh_stride = 0;
    a.block_stride = static_cast<int64_t>(gqla::kBlock) * dq;
    a.kv_off = 0;
    a.k_own = dq;
    a.k_ts = dq;
    a.k_fs = 1;
    a.k_slab = 0;
    a.v_off = 0;
    a.v_half = gqla::kHalf * dq;
    a.v_ts = dq;
    a.v_fs = 1;
  }
  if (pl.n_split > 1) {
    a.ws_o = static_cast<float*>(ws);
    a.ws_lse = a.ws_o + static_cast<size_t>(rows) * pl.n_split * a.dvo;
  }
  a.out = out;
  a.out_kind = out_kind;
  a.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = d->dtype == GQLA_BF16;
  hipError_t e;
  if (pl.tuned) {
    e = gqa ? gqla::launch_tuned_gqa(a, d, s) : gqla::launch_tuned_absorb(a, d, s);
  } else {
    if (gqla::generic_attn_lds_bytes(a.dk, a.dvo) > 160 * 1024)
      return fail(GQLA_ERR_UNSUPPORTED, "key width %d + value width %d exceed the generic kernel's LDS budget", a.dk, a.dvo);
    e = gqla::launch_generic_attn(a, bf16, s);
  }
  if (e != hipSuccess) return hip_fail(e, gqa ? "gqa split-KV decode launch" : "absorb split-KV decode launch");
  if (pl.n_split > 1 && !skip_combine) {
    gqla::CombineParams c{a.ws_o, a.ws_lse, rows, pl.n_split, a.dvo, out, out_kind, lse};
    e = gqla::launch_combine(c, s);
    if (e != hipSuccess) return hip_fail(e, "split-KV combine launch");
  }
  return GQLA_OK;
}

gqla::ProjParams proj_params(const gqla_dims* d) {
  gqla::ProjParams p{};
  p.rows = d->batch * d->s_q;
  p.H = d->num_heads;
  p.G = d->num_groups;
  p.dc = d->latent_rank;
  p.dr = d->rope_dim;
  p.dn = d->nope_dim;
  p.dv = d->v_dim;
  p.rope_shared = d->rope_shared;
  return p;
}

}  // namespace

extern "C" {

gqla_status gqla_absorb_query(const gqla_dims* dims, const void* q_nope, const void* q_rope,
                              const void* w_uk, void* q_abs, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (!q_nope || !w_uk || !q_abs || (dims->rope_dim > 0 && !q_rope))
    return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  const gqla::ProjParams p = proj_params(dims);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gqla::tuned_absorb_query_supported(dims)
                     ? gqla::launch_tuned_absorb_query(p, q_nope, q_rope, w_uk, q_abs, s)
                     : gqla::launch_generic_absorb_query(p, q_nope, q_rope, w_uk, q_abs, dims->dtype == GQLA_BF16, s);
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "absorb query launch");
}

gqla_status gqla_decode_absorb(const gqla_dims* dims, const gqla_paged* paged, const void* q_abs,
                               const void* latent_cache, void* workspace, size_t workspace_bytes,
                               float* o_lat, float* lse, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_paged(dims, paged)) != GQLA_OK) return st;
  if (!q_abs || !latent_cache || !o_lat) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  return run_decode(dims, paged, GQLA_PATH_ABSORB, q_abs, latent_cache, workspace, workspace_bytes,
                    o_lat, gqla::OUT_F32, lse, stream);
}

gqla_status gqla_decode_absorb_out(const gqla_dims* dims, const gqla_paged* paged, const void* q_abs,
                                   const void* latent_cache, const void* w_uv, void* workspace,
                                   size_t workspace_bytes, float* o_lat, void* out, float* lse, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_paged(dims, paged)) != GQLA_OK) return st;
  if (!q_abs || !latent_cache || !w_uv || !o_lat || !out) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  const Plan pl = plan(dims, paged, GQLA_PATH_ABSORB);
  if (!(pl.tuned && gqla::tuned_combine_out_supported(dims, pl.n_split))) {
    // unsplit (the decode writes o_lat itself) or shapes without the fused kernel
    if ((st = gqla_decode_absorb(dims, paged, q_abs, latent_cache, workspace, workspace_bytes, o_lat, lse, stream)) !=
        GQLA_OK)
      return st;
    return gqla_out_proj(dims, o_lat, w_uv, out, stream);
  }
  if ((st = run_decode(dims, paged, GQLA_PATH_ABSORB, q_abs, latent_cache, workspace, workspace_bytes, o_lat,
                       gqla::OUT_F32, lse, stream, true)) != GQLA_OK)
    return st;
  const size_t rows = static_cast<size_t>(dims->batch) * dims->s_q * dims->num_heads;
  const float* ws_o = static_cast<const float*>(workspace);
  const float* ws_lse = ws_o + rows * pl.n_split * dims->latent_rank;
  hipError_t e = gqla::launch_tuned_combine_out(proj_params(dims), ws_o, ws_lse, pl.n_split, o_lat, lse, w_uv, out,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "fused combine and value projection launch");
}

gqla_status gqla_out_proj(const gqla_dims* dims, const float* o_lat, const void* w_uv, void* out,
                          void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (!o_lat || !w_uv || !out) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  const gqla::ProjParams p = proj_params(dims);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gqla::tuned_out_proj_supported(dims)
                     ? gqla::launch_tuned_out_proj(p, o_lat, w_uv, out, s)
                     : gqla::launch_generic_out_proj(p, o_lat, w_uv, out, dims->dtype == GQLA_BF16, s);
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "out projection launch");
}

gqla_status gqla_expand_cache(const gqla_dims* dims, const void* latent_cache, const void* w_uk,
                              const void* w_uv, const int32_t* block_ids, int64_t n_blocks,
                              int64_t num_blocks, void* expanded_cache, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (n_blocks < 0 || num_blocks < 1) return fail(GQLA_ERR_INVALID_ARG, "n_blocks must be >= 0 and num_blocks >= 1");
  if (n_blocks > 0x7fffffff) return fail(GQLA_ERR_INVALID_ARG, "at most 2^31 - 1 blocks per call");
  if (n_blocks == 0) return GQLA_OK;
  if (!latent_cache || !w_uk || !w_uv || !block_ids || !expanded_cache)
    return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  const gqla::ProjParams p = proj_params(dims);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gqla::tuned_expand_supported(dims)
                     ? gqla::launch_tuned_expand(p, latent_cache, w_uk, w_uv, block_ids, n_blocks, num_blocks, expanded_cache, s)
                     : gqla::launch_generic_expand(p, latent_cache, w_uk, w_uv, block_ids, n_blocks, num_blocks,
                                                   expanded_cache, dims->dtype == GQLA_BF16, s);
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "cache expansion launch");
}

gqla_status gqla_decode_gqa(const gqla_dims* dims, const gqla_paged* paged, const void* q,
                            const void* expanded_cache, void* workspace, size_t workspace_bytes,
                            void* out, float* lse, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_paged(dims, paged)) != GQLA_OK) return st;
  if (!q || !expanded_cache || !out) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  return run_decode(dims, paged, GQLA_PATH_GQA, q, expanded_cache, workspace, workspace_bytes, out,
                    dims->dtype == GQLA_BF16 ? gqla::OUT_BF16 : gqla::OUT_F32, lse, stream);
}

gqla_status gqla_num_splits(const gqla_dims* dims, const gqla_paged* paged, int32_t path, int32_t* n) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_path(path)) != GQLA_OK) return st;
  if (n == nullptr) return fail(GQLA_ERR_INVALID_ARG, "n is NULL");
  if (paged == nullptr) return fail(GQLA_ERR_INVALID_ARG, "paged is NULL");
  gqla_paged tmp = *paged;  // only the host-known fields matter here
  tmp.block_table = reinterpret_cast<const int32_t*>(1);
  tmp.ctx_lens = reinterpret_cast<const int32_t*>(1);
  if ((st = check_paged(dims, &tmp)) != GQLA_OK) return st;
  *n = plan(dims, &tmp, path).n_split;
  return GQLA_OK;
}

gqla_status gqla_workspace_bytes(const gqla_dims* dims, const gqla_paged* paged, int32_t path,
                                 size_t* bytes) {
  int32_t n = 0;
  if (bytes == nullptr) return fail(GQLA_ERR_INVALID_ARG, "bytes is NULL");
  gqla_status st = gqla_num_splits(dims, paged, path, &n);
  if (st != GQLA_OK) return st;
  *bytes = workspace_for(dims, path, n);
  return GQLA_OK;
}

int64_t gqla_cache_bytes_per_token(const gqla_dims* dims, int32_t path) {
  if (check_dims(dims) != GQLA_OK || check_path(path) != GQLA_OK) return 0;
  const int64_t elt = elt_bytes(dims);
  if (path == GQLA_PATH_ABSORB) return (dims->latent_rank + dims->rope_dim) * elt;
  return gqla::expanded_layout(dims->nope_dim, dims->rope_dim, dims->v_dim, dims->num_groups, dims->rope_shared != 0).block /
         gqla::kBlock * elt;
}

gqla_status gqla_validate_paged(const gqla_dims* dims, const gqla_paged* paged, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_paged(dims, paged)) != GQLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> lens(dims->batch);
  std::vector<int32_t> table(static_cast<size_t>(dims->batch) * paged->max_blocks_per_seq);
  hipError_t e = hipMemcpyAsync(lens.data(), paged->ctx_lens, lens.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(table.data(), paged->block_table, table.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading paged metadata");
  for (int b = 0; b < dims->batch; ++b) {
    const int L = lens[b];
    if (L < dims->s_q || L > paged->max_ctx_len)
      return fail(GQLA_ERR_INVALID_ARG, "ctx_lens[%d] = %d outside [s_q = %d, max_ctx_len = %d]", b, L,
                  dims->s_q, paged->max_ctx_len);
    for (int k = 0; k < (L + gqla::kBlock - 1) / gqla::kBlock; ++k) {
      const int32_t id = table[static_cast<size_t>(b) * paged->max_blocks_per_seq + k];
      if (id < 0 || id >= paged->num_blocks)
        return fail(GQLA_ERR_INVALID_ARG, "block_table[%d][%d] = %d outside [0, %lld)", b, k, id,
                    static_cast<long long>(paged->num_blocks));
    }
  }
  return GQLA_OK;
}

const char* gqla_status_string(gqla_status status) {
  switch (status) {
    case GQLA_OK: return "ok";
    case GQLA_ERR_INVALID_ARG: return "invalid argument";
    case GQLA_ERR_UNSUPPORTED: return "unsupported dimensions";
    case GQLA_ERR_WORKSPACE: return "workspace too small";
    case GQLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gqla_last_error(void) { return g_err.c_str(); }

const char* gqla_version(void) { return "gqla-mi355x 0.1 (gfx950)"; }

gqla_status gqla_pick_path(const gqla_dims* dims, int64_t total_ctx, int32_t max_ctx, int32_t* path, float* est_us) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (path == nullptr) return fail(GQLA_ERR_INVALID_ARG, "path is NULL");
  if (max_ctx < dims->s_q) return fail(GQLA_ERR_INVALID_ARG, "max_ctx (%d) must be >= s_q (%d)", max_ctx, dims->s_q);
  if (total_ctx < static_cast<int64_t>(dims->batch) * dims->s_q ||
      total_ctx > static_cast<int64_t>(dims->batch) * max_ctx)
    return fail(GQLA_ERR_INVALID_ARG, "total_ctx (%lld) must lie in [batch * s_q, batch * max_ctx]",
                static_cast<long long>(total_ctx));
  gqla_paged pg{};
  pg.max_ctx_len = max_ctx;
  pg.max_blocks_per_seq = (max_ctx + gqla::kBlock - 1) / gqla::kBlock;
  pg.num_blocks = 1;
  const gqla::PathEstimate e =
      gqla::estimate_paths(dims, total_ctx, plan(dims, &pg, GQLA_PATH_ABSORB).n_split, plan(dims, &pg, GQLA_PATH_GQA).n_split);
  *path = e.gqa_us < e.absorb_us ? GQLA_PATH_GQA : GQLA_PATH_ABSORB;
  if (est_us != nullptr) {
    est_us[0] = static_cast<float>(e.absorb_us);
    est_us[1] = static_cast<float>(e.gqa_us);
  }
  return GQLA_OK;
}

gqla_status gqla_append_tokens(const gqla_dims* dims, const gqla_paged* paged, const void* c_new,
                               const void* kr_new, float rope_theta, const void* w_uk, const void* w_uv,
                               void* latent_cache, void* expanded_cache, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if ((st = check_paged(dims, paged)) != GQLA_OK) return st;
  if (!c_new || (dims->rope_dim > 0 && !kr_new))
    return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  if (!latent_cache && !expanded_cache)
    return fail(GQLA_ERR_INVALID_ARG, "latent_cache and expanded_cache are both NULL: nothing to write");
  if (expanded_cache && (!w_uk || !w_uv)) return fail(GQLA_ERR_INVALID_ARG, "expansion needs w_uk and w_uv");
  if (!(rope_theta > 0.f)) return fail(GQLA_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (dims->rope_dim % 2 != 0) return fail(GQLA_ERR_INVALID_ARG, "rope_dim must be even (rotation pairs)");
  if (dims->latent_rank % 8 != 0) return fail(GQLA_ERR_UNSUPPORTED, "append needs latent_rank % 8 == 0");
  if (dims->rope_dim > 128) return fail(GQLA_ERR_UNSUPPORTED, "append supports rope_dim <= 128");
  if (static_cast<int64_t>(16) * (dims->latent_rank + dims->rope_dim) * 4 > 160 * 1024)
    return fail(GQLA_ERR_UNSUPPORTED, "latent row too wide for the append kernel's LDS tile");
  const int64_t n_tok = static_cast<int64_t>(dims->batch) * dims->s_q;
  if (n_tok > 0x7fffffff) return fail(GQLA_ERR_INVALID_ARG, "too many new tokens");
  gqla::AppendParams a{};
  a.block_table = paged->block_table;
  a.ctx_lens = paged->ctx_lens;
  a.max_blocks = paged->max_blocks_per_seq;
  a.num_blocks = paged->num_blocks;
  a.n_tok = static_cast<int32_t>(n_tok);
  a.s_q = dims->s_q;
  a.G = dims->num_groups;
  a.dc = dims->latent_rank;
  a.dr = dims->rope_dim;
  a.dn = dims->nope_dim;
  a.dv = dims->v_dim;
  a.rope_shared = dims->rope_shared;
  a.rope_theta = rope_theta;
  for (int k = 0; k < dims->rope_dim / 2; ++k)
    a.inv_freq[k] = std::pow(static_cast<double>(rope_theta), -2.0 * k / dims->rope_dim);
  hipError_t e = gqla::launch_append(a, c_new, kr_new, w_uk, w_uv, latent_cache, expanded_cache,
                                     dims->dtype == GQLA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "append launch");
}

gqla_status gqla_out_hidden(const gqla_dims* dims, int32_t hidden, int32_t folded, const void* x,
                            const void* w, void* y, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (hidden < 1 || hidden > 65535) return fail(GQLA_ERR_INVALID_ARG, "hidden must be in [1, 65535], got %d", hidden);
  if (folded != 0 && folded != 1) return fail(GQLA_ERR_INVALID_ARG, "folded must be 0 or 1");
  if (!x || !w || !y) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  const int64_t rows = static_cast<int64_t>(dims->batch) * dims->s_q;
  const int64_t k = static_cast<int64_t>(dims->num_heads) * (folded ? dims->latent_rank : dims->v_dim);
  if (rows > 0x7fffffff || k > 0x7fffffff) return fail(GQLA_ERR_INVALID_ARG, "output side too large");
  const bool bf16 = dims->dtype == GQLA_BF16;
  hipError_t e = gqla::launch_out_hidden(x, folded == 1 || !bf16, w, y, static_cast<int>(rows), hidden,
                                         static_cast<int>(k), bf16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "output projection launch");
}

gqla_status gqla_fold_out_weight(const gqla_dims* dims, int32_t hidden, const void* w_o, const void* w_uv,
                                 void* w_fold, void* stream) {
  gqla_status st = check_dims(dims);
  if (st != GQLA_OK) return st;
  if (hidden < 1 || hidden > 65535) return fail(GQLA_ERR_INVALID_ARG, "hidden must be in [1, 65535], got %d", hidden);
  if (!w_o || !w_uv || !w_fold) return fail(GQLA_ERR_INVALID_ARG, "null tensor pointer");
  hipError_t e = gqla::launch_fold_out_weight(proj_params(dims), hidden, w_o, w_uv, w_fold, dims->dtype == GQLA_BF16,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQLA_OK : hip_fail(e, "weight fold launch");
}

}  // extern "C"
