"""Test-side plumbing for the GPU parity tests: upload seeded inputs with torch, call the
HIP path through the C ABI binding, and compute the matching oracle results."""
import sys

import numpy as np
import torch

from oracle import gqla_ref as R

TOL = {"bf16": 1e-2, "f32": 1e-5}   # max|gpu - ref| <= TOL * max|ref|


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        u = t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return t.double().numpy()


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class Run:
    """Device copies of one Inputs batch and calls of both GQLA paths."""

    def __init__(self, x, num_splits: int = 0, rope_shared: bool = False):
        import decode_attention_02_amd as G
        self.G = G
        self.x = x
        self.rope_shared = rope_shared
        w = x.w
        self.dims = G.Dims(batch=len(x.ctx_lens), num_heads=w.heads, num_groups=w.groups,
                           latent_rank=w.latent, rope_dim=w.rope, nope_dim=w.nope, v_dim=w.v,
                           s_q=x.s_q, dtype=G.GQLA_BF16 if x.dtype == "bf16" else G.GQLA_F32,
                           rope_shared=int(rope_shared))
        self.cache = to_dev(x.latent_cache, x.dtype)
        self.w_uk = to_dev(x.w_uk, x.dtype)
        self.w_uv = to_dev(x.w_uv, x.dtype)
        self.q_nope = to_dev(x.q_nope, x.dtype)
        self.q_rope = to_dev(x.q_rope, x.dtype)
        self.q = to_dev(x.q, x.dtype)
        self.table = torch.from_numpy(x.block_table).cuda()
        self.lens = torch.from_numpy(x.ctx_lens).cuda()
        self.paged = G.Paged(self.table, self.lens, int(x.ctx_lens.max()), x.num_blocks, num_splits)
        self.B = len(x.ctx_lens)

    def workspace(self, path):
        G = self.G
        n = G.gqla_workspace_bytes(self.dims, path, self.table.shape[1], self.paged.max_ctx_len,
                                   self.paged.num_blocks, self.paged.num_splits)
        return torch.empty(max(n, 4) // 4, dtype=torch.float32, device="cuda") if n else None

    def absorb(self):
        G, w, x = self.G, self.x.w, self.x
        dt = torch_dtype(x.dtype)
        q_abs = torch.full((self.B, x.s_q, w.heads, w.latent + w.rope), float("nan"), dtype=dt, device="cuda")
        o_lat = torch.full((self.B, x.s_q, w.heads, w.latent), float("nan"), device="cuda")
        lse = torch.full((self.B, x.s_q, w.heads), float("nan"), device="cuda")
        out = torch.full((self.B, x.s_q, w.heads, w.v), float("nan"), dtype=dt, device="cuda")
        G.gqla_absorb_query(self.dims, self.q_nope, self.q_rope, self.w_uk, q_abs)
        G.gqla_decode_absorb(self.dims, self.paged, q_abs, self.cache, self.workspace(G.GQLA_PATH_ABSORB), o_lat, lse)
        G.gqla_out_proj(self.dims, o_lat, self.w_uv, out)
        torch.cuda.synchronize()
        return dict(q_abs=to_host(q_abs), o_lat=to_host(o_lat), lse=to_host(lse), out=to_host(out))

    def expand(self, block_ids=None):
        G, w, x = self.G, self.x.w, self.x
        dt = torch_dtype(x.dtype)
        per_block = expanded_block_values(w.groups, w.qk, w.v, self.rope_shared, w.rope)
        expanded = torch.full((x.num_blocks * per_block,), float("nan"), dtype=dt, device="cuda")
        ids = torch.arange(x.num_blocks, dtype=torch.int32, device="cuda") if block_ids is None else block_ids
        G.gqla_expand_cache(self.dims, self.cache, self.w_uk, self.w_uv, ids, x.num_blocks, expanded)
        return expanded

    def gqa(self, expanded=None):
        G, w, x = self.G, self.x.w, self.x
        dt = torch_dtype(x.dtype)
        if expanded is None:
            expanded = self.expand()
        out = torch.full((self.B, x.s_q, w.heads, w.v), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((self.B, x.s_q, w.heads), float("nan"), device="cuda")
        G.gqla_decode_gqa(self.dims, self.paged, self.q, expanded, self.workspace(G.GQLA_PATH_GQA), out, lse)
        torch.cuda.synchronize()
        return dict(out=to_host(out), lse=to_host(lse), expanded=expanded)


def _slab_widths(n: int):
    return [min(32, n - s) for s in range(0, n, 32)]


def _slabs_to_logical(a: np.ndarray, n_feat: int) -> np.ndarray:
    """[..., 64 * n_feat] in 32-feature slabs ([64][w] each) -> [..., 64, n_feat]."""
    parts, off = [], 0
    for w in _slab_widths(n_feat):
        parts.append(a[..., off:off + 64 * w].reshape(a.shape[:-1] + (64, w)))
        off += 64 * w
    return np.concatenate(parts, axis=-1)


def _logical_to_slabs(a: np.ndarray) -> np.ndarray:
    """[..., 64, n_feat] -> [..., 64 * n_feat] in 32-feature slabs."""
    n_feat = a.shape[-1]
    parts, s = [], 0
    for w in _slab_widths(n_feat):
        parts.append(a[..., s:s + w].reshape(a.shape[:-2] + (-1,)))
        s += w
    return np.concatenate(parts, axis=-1)


def expanded_block_values(G: int, dqk: int, dv: int, rope_shared: bool = False, dr: int = 0) -> int:
    """Values per 64-token block of the expanded cache (both layouts)."""
    return 64 * (dr + G * (dqk - dr + dv)) if rope_shared else 64 * G * (dqk + dv)


def expanded_to_logical(flat: np.ndarray, num_blocks: int, G: int, dqk: int, dv: int,
                        rope_shared: bool = False, dr: int = 0):
    """Read the documented expanded-cache layout back into K [NB][G][64][dqk] and
    V [NB][G][64][dv] (token-major) for comparison. Per (block, group) chunk: K as
    slabs of 32 features, each [64 slots][width]; then V as two 32-slot halves, each
    [dv][32]. With rope_shared the block starts with the RoPE keys once (slabs over d_R)
    and each group chunk holds only the d_n key features; K is returned with the shared
    key repeated in every group."""
    blk = flat.reshape(num_blocks, expanded_block_values(G, dqk, dv, rope_shared, dr))
    kf = dqk - dr if rope_shared else dqk
    rope_vals = 64 * dr if rope_shared else 0
    chunk = blk[:, rope_vals:].reshape(num_blocks, G, 64 * (kf + dv))
    K = _slabs_to_logical(chunk[:, :, :64 * kf], kf)
    if rope_shared:
        rk = _slabs_to_logical(blk[:, :rope_vals], dr)
        K = np.concatenate([K, np.repeat(rk[:, None], G, axis=1)], axis=-1)
    V = chunk[:, :, 64 * kf:].reshape(num_blocks, G, 2, dv, 32).transpose(0, 1, 2, 4, 3).reshape(num_blocks, G, 64, dv)
    return K, V


def logical_to_expanded(K: np.ndarray, V: np.ndarray, rope_shared: bool = False, dr: int = 0) -> np.ndarray:
    """Inverse of expanded_to_logical (with rope_shared, the shared key is group 0's)."""
    NB, G, _, dqk = K.shape
    dv = V.shape[3]
    kf = dqk - dr if rope_shared else dqk
    Vh = V.reshape(NB, G, 2, 32, dv).transpose(0, 1, 2, 4, 3).reshape(NB, G, -1)
    chunks = np.concatenate([_logical_to_slabs(K[..., :kf]), Vh], axis=2).reshape(NB, -1)
    if rope_shared:
        chunks = np.concatenate([_logical_to_slabs(K[:, 0, :, kf:]), chunks], axis=1)
    return chunks.reshape(-1)


def oracle_paths(x, seqs=None):
    """Oracle results for the listed sequences: naive (definition), absorb and gqa."""
    w = x.w
    f = x.f64
    seqs = list(range(len(x.ctx_lens))) if seqs is None else list(seqs)
    sc = R.qk_scale(w.nope, w.rope)
    c = {b: f(x.c_kv_seq[b]) for b in seqs}
    kr = {b: f(x.k_rope_seq[b]) for b in seqs}
    wk, wv = f(x.w_uk), f(x.w_uv)
    res = {}
    for b in seqs:
        qn, qr = f(x.q_nope[b]), f(x.q_rope[b])
        out, lse = R.mla_expanded_attention(c[b], kr[b], wk, wv, qn, qr, x.s_q, sc)
        q_abs = R.absorb_query(qn, qr, wk)
        o_lat, alse = R.absorb_attention(q_abs, c[b], kr[b], x.s_q, sc)
        res[b] = dict(out=out, lse=lse, q_abs=q_abs, o_lat=o_lat, absorb_lse=alse,
                      absorb_out=R.out_projection(o_lat, wv))
    return res


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.isfinite(got).all():
        return float("inf")
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
