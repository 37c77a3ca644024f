"""Seeded input generation for GQLA decode workloads.

Recipe (one stream per tensor, spawned from SeedSequence(workload.seed) in a fixed order:
latent c_KV, RoPE keys, W_UK, W_UV, q_nope, q_rope, context lengths, block permutation;
the two cache streams spawn one child per sequence so any sequence can be regenerated
alone):

* c_KV and k_rope ~ N(0, 1) per token; k_rope of token t is rotated to position t.
* W_UK^g [d_n][d_c] and W_UV^g [d_v][d_c] ~ N(0, std = 1/sqrt(d_c)) (fan_in = d_c).
* q_nope, q_rope ~ N(0, 1); q_rope of row i is rotated to position L_b - s_q + i.
* RoPE uses theta = 10000 and the half-split pairing (x[k], x[k + d_R/2]).
* Everything is rounded once to the storage dtype (round-to-nearest-even for bf16).
* Context lengths are fixed, or integer-uniform in [lo, hi] inclusive.
* Logical token t of sequence b lives at physical (block_table[b][t // 64], t % 64).
  The block table is the identity layout, or a seeded permutation of all pool blocks.
  Cache slots past a sequence's end are filled with NaN, and unused block-table entries
  are -1, so a reader that strays past the context shows up in the results.
"""
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .shapes import Workload

BLOCK = 64
ROPE_THETA = 10000.0
BF16_NAN = np.uint16(0x7FC0)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest, ties to even) via fp32, returning the 16-bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate the last axis of x (size d_R, even) to the given positions.

    Half-split pairing: component k is paired with k + d_R/2 and rotated by the angle
    position * theta**(-2k/d_R). positions broadcasts against x.shape[:-1].
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


@dataclass
class Inputs:
    """One seeded batch. Storage arrays hold bf16 bit patterns (uint16) or float32."""
    w: Workload
    s_q: int
    dtype: str
    ctx_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B][max_blocks], -1 where unused
    num_blocks: int
    latent_cache: np.ndarray      # [num_blocks][64][d_c + d_R]
    w_uk: np.ndarray              # [G][d_n][d_c]
    w_uv: np.ndarray              # [G][d_v][d_c]
    q_nope: np.ndarray            # [B][s_q][H][d_n]
    q_rope: np.ndarray            # [B][s_q][H][d_R]
    c_kv_seq: List[np.ndarray]    # per sequence [L_b][d_c], storage dtype (logical order)
    k_rope_seq: List[np.ndarray]  # per sequence [L_b][d_R], storage dtype (logical order)

    def f64(self, a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f64(a) if self.dtype == "bf16" else np.asarray(a, np.float64)

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def q(self) -> np.ndarray:
        """GQA-path query [B][s_q][H][d_n + d_R] = [q_nope | q_rope] (storage dtype)."""
        return np.concatenate([self.q_nope, self.q_rope], axis=-1)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f64_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def _nan(dtype: str):
    return BF16_NAN if dtype == "bf16" else np.float32(np.nan)


def generate(w: Workload, s_q: int, *, batch: Optional[int] = None,
             ctx_lens: Optional[Sequence[int]] = None, dtype: Optional[str] = None,
             shuffled: Optional[bool] = None, extra_blocks: int = 0,
             seed: Optional[int] = None) -> Inputs:
    """Materialise one batch of workload w at s_q query rows per sequence.

    batch / ctx_lens / dtype / shuffled override the workload (used for small parity
    cases at the workload's head dimensions). extra_blocks adds unused pool blocks.
    """
    B = batch if batch is not None else w.batch
    dt = dtype or w.dtype
    shuf = w.shuffled if shuffled is None else shuffled
    H, G, dc, dr, dn, dv = w.heads, w.groups, w.latent, w.rope, w.nope, w.v
    streams = np.random.SeedSequence(w.seed if seed is None else seed).spawn(8)
    ss_c, ss_r, ss_wk, ss_wv, ss_qn, ss_qr, ss_len, ss_perm = streams

    if ctx_lens is None:
        lo, hi = w.ctx
        if lo == hi:
            lens = np.full(B, lo, dtype=np.int64)
        else:
            lens = np.random.default_rng(ss_len).integers(lo, hi + 1, size=B)
    else:
        lens = np.asarray(ctx_lens, dtype=np.int64)
        assert lens.shape == (B,)
    if (lens < s_q).any():
        raise ValueError("every context must hold at least the s_q new tokens")

    nblk = (lens + BLOCK - 1) // BLOCK
    num_blocks = int(nblk.sum()) + extra_blocks
    max_blocks = int(nblk.max())
    if shuf:
        phys = np.random.default_rng(ss_perm).permutation(num_blocks)
    else:
        phys = np.arange(num_blocks)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        table[b, :nblk[b]] = phys[start:start + nblk[b]]
        start += nblk[b]

    cache_dtype = np.uint16 if dt == "bf16" else np.float32
    cache = np.empty((num_blocks, BLOCK, dc + dr), dtype=cache_dtype)
    cache[...] = _nan(dt)

    c_children = ss_c.spawn(B)
    r_children = ss_r.spawn(B)
    c_seq, r_seq = [], []
    for b in range(B):
        L = int(lens[b])
        c = np.random.default_rng(c_children[b]).standard_normal((L, dc))
        kr = np.random.default_rng(r_children[b]).standard_normal((L, dr))
        kr = rope_rotate(kr, np.arange(L))
        cs, rs = _store(c, dt), _store(kr, dt)
        c_seq.append(cs)
        r_seq.append(rs)
        t = np.arange(L)
        blk = table[b, t // BLOCK]
        cache[blk, t % BLOCK, :dc] = cs
        cache[blk, t % BLOCK, dc:] = rs

    std = 1.0 / np.sqrt(dc)
    w_uk = _store(np.random.default_rng(ss_wk).standard_normal((G, dn, dc)) * std, dt)
    w_uv = _store(np.random.default_rng(ss_wv).standard_normal((G, dv, dc)) * std, dt)
    q_nope, q_rope = _queries(w, s_q, lens, ss_qn, ss_qr, dt)
    return Inputs(w=w, s_q=s_q, dtype=dt, ctx_lens=lens.astype(np.int32),
                  block_table=table, num_blocks=num_blocks, latent_cache=cache,
                  w_uk=w_uk, w_uv=w_uv, q_nope=q_nope, q_rope=q_rope,
                  c_kv_seq=c_seq, k_rope_seq=r_seq)


def _queries(w: Workload, s_q: int, lens: np.ndarray, ss_qn, ss_qr, dt: str):
    B, H = len(lens), w.heads
    q_nope = np.random.default_rng(ss_qn).standard_normal((B, s_q, H, w.nope))
    q_rope = np.random.default_rng(ss_qr).standard_normal((B, s_q, H, w.rope))
    pos = np.asarray(lens)[:, None] - s_q + np.arange(s_q)[None, :]   # [B][s_q]
    q_rope = rope_rotate(q_rope, pos[:, :, None])
    return _store(q_nope, dt), _store(q_rope, dt)


def queries_for(x: Inputs, s_q: int, seed: Optional[int] = None):
    """Queries of batch x at another s_q (same seed streams, same context lengths):
    returns (q_nope, q_rope) in the storage dtype."""
    streams = np.random.SeedSequence(x.w.seed if seed is None else seed).spawn(8)
    return _queries(x.w, s_q, x.ctx_lens.astype(np.int64), streams[4], streams[5], x.dtype)
