"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark
times (automatic split plan), on sampled sequences the oracle computes one by one, plus
properties that hold at any size (finite outputs, both paths agree on every sequence)."""
import ctypes
import time

import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from decode_attention_02_amd import _lib
from workloads import generate, workload

from gpu_util import TOL, Run, log, oracle_paths, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def _compare(x, got_a, got_g, seqs, label):
    ref = oracle_paths(x, seqs)
    for b in seqs:
        r = ref[b]
        ea, eg = rel_err(got_a["out"][b], r["out"]), rel_err(got_g["out"][b], r["out"])
        el = rel_err(got_a["o_lat"][b], r["o_lat"])
        la = float(np.max(np.abs(got_a["lse"][b] - r["lse"])))
        lg = float(np.max(np.abs(got_g["lse"][b] - r["lse"])))
        log(f"  {label} seq {b} L={int(x.ctx_lens[b])}: absorb {ea:.2e} gqa {eg:.2e} o_lat {el:.2e} "
            f"lse {la:.1e}/{lg:.1e}")
        lse_tol = TOL["bf16"] * max(1.0, float(np.max(np.abs(r["lse"]))))
        assert ea <= TOL["bf16"] and eg <= TOL["bf16"] and el <= TOL["bf16"]
        assert la <= lse_tol and lg <= lse_tol


@pytest.mark.parametrize("name,s_q,rope_shared", [("llama3-8b-b32-ctx8k", 1, False), ("llama3-8b-b32-ctx8k", 2, False),
                                                  ("dsv3-b64-ctx8k", 1, False), ("dsv3-b64-ctx8k", 2, False),
                                                  ("dsv3-b8-ctx32k-64k", 2, False), ("llama3-8b-b32-ctx8k", 2, True),
                                                  ("dsv3-b8-ctx32k-64k", 2, True)])
def test_fullsize_sampled(name, s_q, rope_shared):
    w = workload(name)
    log(f"fullsize {name} s_q={s_q} rope_shared={rope_shared}: generating")
    x = generate(w, s_q)
    B = len(x.ctx_lens)
    run = Run(x, 0, rope_shared)
    log(f"fullsize {name} s_q={s_q}: running both paths (B={B}, max ctx {int(x.ctx_lens.max())})")
    got_a, got_g = run.absorb(), run.gqa()
    del run
    torch.cuda.empty_cache()
    assert np.isfinite(got_a["out"]).all() and np.isfinite(got_g["out"]).all()
    assert np.isfinite(got_a["lse"]).all() and np.isfinite(got_g["lse"]).all()
    assert rel_err(got_a["out"], got_g["out"]) <= TOL["bf16"]
    # every sequence of a batch of at most 8 (the long-context batch: all its lengths and
    # split boundaries); else the first, the last, and the shortest, a median and the
    # longest context of the batch
    if B <= 8:
        seqs = list(range(B))
    else:
        order = np.argsort(x.ctx_lens, kind="stable")
        seqs = sorted({0, B - 1, int(order[0]), int(order[B // 2]), int(order[-1])})
    _compare(x, got_a, got_g, seqs, name)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_tp8share_capacity_fullsize_sampled():
    """The one-eighth DeepSeek-V3 head share at batch 10240 x context 16384: the expanded
    cache alone fills 200 GiB, so the latent is generated and expanded in chunks, the GQA
    decode runs over the whole pool, then the same latent is regenerated for the absorb
    path. Sequences 0..15 carry the workload recipe's host-generated data and are checked
    against the oracle; every sequence must agree between the two paths."""
    w = workload("dsv3-tp8share-ctx16k")
    s_q, B, L = 2, w.batch, w.ctx[0]
    nbs = L // 64
    NB = B * nbs
    n_sample = 16
    blk_bytes = 64 * (w.latent + w.rope) * 2
    log(f"capacity: B={B} L={L} NB={NB}; host data for {n_sample} sequences")
    xs = generate(w, s_q, batch=n_sample, ctx_lens=[L] * n_sample, shuffled=False)
    perm = np.random.default_rng(w.seed).permutation(NB).astype(np.int32)
    table_h = perm.reshape(B, nbs)
    table = torch.from_numpy(table_h).cuda()
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    w_uk, w_uv = to_dev(xs.w_uk, "bf16"), to_dev(xs.w_uv, "bf16")
    gen = torch.Generator(device="cuda")

    def randn(shape, seed):
        gen.manual_seed(seed)
        return torch.randn(shape, generator=gen, device="cuda", dtype=torch.bfloat16)

    q = randn((B, s_q, w.heads, w.qk), 11)
    q[:n_sample] = to_dev(xs.q, "bf16")
    q_nope = q[..., :w.nope].contiguous()
    q_rope = q[..., w.nope:].contiguous()
    sample_blocks = table_h[:n_sample].reshape(-1)               # physical ids of sampled data
    sample_rows = torch.from_numpy(np.ascontiguousarray(xs.latent_cache.view(np.int16))).view(torch.bfloat16)
    sample_src = np.arange(n_sample * nbs)                       # their blocks in xs (identity)
    n_chunks = 32
    chunk = (NB + n_chunks - 1) // n_chunks

    def latent_chunk(c):
        lo, hi = c * chunk, min(NB, (c + 1) * chunk)
        t = randn((hi - lo, 64, w.latent + w.rope), 1000 + c)
        sel = np.nonzero((sample_blocks >= lo) & (sample_blocks < hi))[0]
        if len(sel):
            dst = torch.from_numpy((sample_blocks[sel] - lo).astype(np.int64)).cuda()
            t[dst] = sample_rows[torch.from_numpy(sample_src[sel])].cuda()
        return lo, hi, t

    dims = G.Dims(batch=B, num_heads=w.heads, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                  nope_dim=w.nope, v_dim=w.v, s_q=s_q)
    dc = dims.c()
    paged = G.Paged(table, lens, L, NB)
    per_block = w.groups * 64 * (w.qk + w.v)
    log(f"capacity: expanded cache {NB * per_block * 2 / 2**30:.1f} GiB")
    expanded = torch.empty(NB * per_block, dtype=torch.bfloat16, device="cuda")
    for c in range(n_chunks):
        lo, hi, t = latent_chunk(c)
        ids = torch.arange(lo, hi, dtype=torch.int32, device="cuda")
        # the pool pointer is shifted so that block id `lo` lands on the chunk's first block;
        # only ids in [lo, hi) are read
        st = _lib.LIB.gqla_expand_cache(ctypes.byref(dc), ctypes.c_void_p(t.data_ptr() - lo * blk_bytes),
                                        _ptr(w_uk), _ptr(w_uv), _ptr(ids), hi - lo, NB, _ptr(expanded),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, _lib.LIB.gqla_last_error()
        torch.cuda.synchronize()
        del t, ids
    log("capacity: GQA decode")
    out_g = torch.empty(B, s_q, w.heads, w.v, dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty(B, s_q, w.heads, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    G.gqla_decode_gqa(dims, paged, q, expanded, None, out_g, lse_g)
    e0.record()
    G.gqla_decode_gqa(dims, paged, q, expanded, None, out_g, lse_g)
    e1.record()
    torch.cuda.synchronize()
    t_g = e0.elapsed_time(e1) / 1e3
    kv_g = B * L * per_block / 64 * 2
    log(f"capacity: GQA decode {t_g * 1e3:.2f} ms, {kv_g / t_g / 1e9:.0f} GB/s, {B * s_q / t_g:.0f} tokens/s")
    del expanded
    torch.cuda.empty_cache()

    log("capacity: absorb path over the regenerated latent")
    latent = torch.empty((NB, 64, w.latent + w.rope), dtype=torch.bfloat16, device="cuda")
    for c in range(n_chunks):
        lo, hi, t = latent_chunk(c)
        latent[lo:hi] = t
        del t
    q_abs = torch.empty(B, s_q, w.heads, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(B, s_q, w.heads, w.latent, device="cuda")
    lse_a = torch.empty(B, s_q, w.heads, device="cuda")
    out_a = torch.empty(B, s_q, w.heads, w.v, dtype=torch.bfloat16, device="cuda")
    G.gqla_absorb_query(dims, q_nope, q_rope, w_uk, q_abs)
    G.gqla_decode_absorb(dims, paged, q_abs, latent, None, o_lat, lse_a)
    e0.record()
    G.gqla_decode_absorb(dims, paged, q_abs, latent, None, o_lat, lse_a)
    e1.record()
    G.gqla_out_proj(dims, o_lat, w_uv, out_a)
    torch.cuda.synchronize()
    t_a = e0.elapsed_time(e1) / 1e3
    kv_a = B * L * (w.latent + w.rope) * 2
    log(f"capacity: absorb decode {t_a * 1e3:.2f} ms, {kv_a / t_a / 1e9:.0f} GB/s, {B * s_q / t_a:.0f} tokens/s")
    del latent
    torch.cuda.empty_cache()

    got_g = dict(out=to_host(out_g), lse=to_host(lse_g))
    got_a = dict(out=to_host(out_a), lse=to_host(lse_a), o_lat=to_host(o_lat[:n_sample]))
    assert np.isfinite(got_g["out"]).all() and np.isfinite(got_a["out"]).all()
    assert rel_err(got_a["out"], got_g["out"]) <= TOL["bf16"]
    _compare(xs, {k: v[:n_sample] for k, v in got_a.items()}, {k: v[:n_sample] for k, v in got_g.items()},
             [0, 7, 15], "capacity")
