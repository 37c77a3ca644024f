"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

No GPU. Each test names the fact it pins. Planted mistakes live in the oracle copies
built by `_mutant` (CPU only) and must make at least one pin fail.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import gqla_ref as R
from workloads import generate, rope_rotate, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64_inputs(x):
    f = x.f64
    return ([f(c) for c in x.c_kv_seq], [f(r) for r in x.k_rope_seq], f(x.w_uk), f(x.w_uv),
            f(x.q_nope), f(x.q_rope), f(x.q))


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(b)))


def _sdpa_bottom_right(q, K, V, s_q, scale, enable_gqa):
    """torch CPU fp64 SDPA with an explicit bottom-right causal mask.
    q [s_q][H][d], K/V [G][L][d] -> [s_q][H][d_v]."""
    L = K.shape[1]
    mask = torch.arange(L)[None, :] <= (L - s_q + torch.arange(s_q))[:, None]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V))[None]
    if not enable_gqa:
        rep = q.shape[1] // K.shape[0]
        kt = kt.repeat_interleave(rep, dim=1)
        vt = vt.repeat_interleave(rep, dim=1)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                       enable_gqa=enable_gqa)
    return o[0].numpy().transpose(1, 0, 2)


# ------------------------------------------------------------------ definition pins

@pytest.mark.parametrize("s_q", [1, 2])
def test_brute_force_matches_definition(s_q):
    """Pure-Python loops (math.exp / math.fsum) agree with the NumPy definition."""
    w = workload("tiny-fp32")
    x = generate(w, s_q)
    c, kr, wk, wv, qn, qr, _ = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    for b in range(w.batch):
        out, lse = R.mla_expanded_attention(c[b], kr[b], wk, wv, qn[b], qr[b], s_q, sc)
        bo, bl = R.brute_mla_attention(c[b], kr[b], wk, wv, qn[b], qr[b], s_q, sc)
        assert _rel(bo, out) < 1e-12
        assert np.max(np.abs(bl - lse)) < 1e-12


@pytest.mark.parametrize("name,s_q,ctx", [("tiny-fp32", 1, None), ("tiny-fp32", 2, None),
                                          ("llama3-8b-b32-ctx8k", 2, [70, 1]),
                                          ("dsv3-b64-ctx8k", 1, [130, 64])])
def test_absorb_path_equals_expanded_form(name, s_q, ctx):
    """MQA-absorb (fold W_UK^g into q, attend over the latent, apply W_UV^g) equals the
    head-expanded MLA form: the two are algebraically equivalent (GQLA abstracts)."""
    w = workload(name)
    kw = {} if ctx is None else dict(batch=len(ctx), ctx_lens=[max(c, s_q) for c in ctx])
    x = generate(w, s_q, **kw)
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    naive = R.batch_naive(c, kr, wk, wv, qn, qr, s_q, sc)
    absorb = R.batch_absorb(c, kr, wk, wv, qn, qr, s_q, sc)
    for (out, lse), (_, _, alse, aout) in zip(naive, absorb):
        assert _rel(aout, out) < 1e-12
        assert np.max(np.abs(alse - lse)) < 1e-12


@pytest.mark.parametrize("name,s_q,ctx", [("tiny-fp32", 1, None), ("tiny-fp32", 2, None),
                                          ("dsv3-b64-ctx8k", 2, [129, 2])])
def test_gqa_path_matches_sdpa(name, s_q, ctx):
    """The GQA step equals torch's scaled_dot_product_attention with enable_gqa and with
    key/value heads copied gs times (the glossary's equivalence), under a bottom-right
    causal mask, in fp64 on the CPU."""
    w = workload(name)
    kw = {} if ctx is None else dict(batch=len(ctx), ctx_lens=ctx)
    x = generate(w, s_q, **kw)
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    for b in range(len(c)):
        K, V = R.expand_latent(c[b], kr[b], wk, wv)
        out, lse = R.gqa_attention(q[b], K, V, s_q, sc)
        assert _rel(_sdpa_bottom_right(q[b], K, V, s_q, sc, True), out) < 1e-12
        assert _rel(_sdpa_bottom_right(q[b], K, V, s_q, sc, False), out) < 1e-12
        # lse against scipy's logsumexp of the visible scores
        for i in range(s_q):
            n = R.visible_tokens(K.shape[1], s_q, i)
            for h in range(q.shape[2]):
                g = R.head_group(h, q.shape[2], K.shape[0])
                ref = logsumexp(sc * (K[g, :n] @ q[b][i, h]))
                assert abs(ref - lse[i, h]) < 1e-12


def _scale_pin_passes(M, name):
    """M's definition and absorb path, each at M.qk_scale(d_n, d_R), against torch SDPA left
    at its DEFAULT scale (no scale= argument: SDPA divides by the square root of the query
    width E, here the non-absorbed head width d_n + d_R of the [q_nope | q_rope] queries).
    The module's constructor fixes the same value (GQLAAttention scales by
    head_dim ** -0.5). The workloads' latent widths d_c + d_R (80, 576) differ from
    d_n + d_R (48, 192), so an absorbed-width scale cannot pass."""
    w = workload(name)
    s_q = 2
    x = generate(w, s_q, batch=1, ctx_lens=[37])
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = M.qk_scale(w.nope, w.rope)
    K, V = R.expand_latent(c[0], kr[0], wk, wv)
    L = K.shape[1]
    mask = torch.arange(L)[None, :] <= (L - s_q + torch.arange(s_q))[:, None]
    rep = w.heads // w.groups
    qt = torch.from_numpy(np.ascontiguousarray(q[0].transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None].repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(V))[None].repeat_interleave(rep, dim=1)
    assert qt.shape[-1] == w.nope + w.rope
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[0].numpy().transpose(1, 0, 2)
    out, _ = M.mla_expanded_attention(c[0], kr[0], wk, wv, qn[0], qr[0], s_q, sc)
    ab = M.batch_absorb(c, kr, wk, wv, qn, qr, s_q, sc)[0][3]
    return _rel(out, ref) < 1e-12 and _rel(ab, ref) < 1e-12


@pytest.mark.parametrize("name", ["tiny-fp32", "dsv3-b64-ctx8k"])
def test_qk_scale_is_sdpa_default_scale(name):
    """Softmax scale pin: qk_scale(d_n, d_R) is the scale torch SDPA applies by default to
    the non-absorbed queries, 1/sqrt(d_n + d_R) (the module's head_dim ** -0.5)."""
    assert _scale_pin_passes(R, name)


@pytest.mark.parametrize("name", ["tiny-fp32", "dsv3-b64-ctx8k"])
def test_scale_pin_catches_absorbed_width_scale(name):
    """Planted mistake: scaling by the absorbed key width, 1/sqrt(d_c + d_R), fails."""
    w = workload(name)
    M = _mutant(qk_scale=lambda d_n, d_r: 1.0 / math.sqrt(w.latent + d_r))
    assert not _scale_pin_passes(M, name)


@pytest.mark.parametrize("s_q", [1, 2])
def test_one_token_context_returns_value_exactly(s_q):
    """With one visible token the softmax weight is exactly 1: out = V_0 and o_lat = c_0
    bit for bit (row 0 at s_q = 2 with a context of 2 tokens sees one token)."""
    w = workload("dsv3-b64-ctx8k")
    x = generate(w, s_q, batch=2, ctx_lens=[s_q, s_q])
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    for b in range(2):
        out, _ = R.mla_expanded_attention(c[b], kr[b], wk, wv, qn[b], qr[b], s_q, sc)
        qa = R.absorb_query(qn[b], qr[b], wk)
        o_lat, _ = R.absorb_attention(qa, c[b], kr[b], s_q, sc)
        K, V = R.expand_latent(c[b], kr[b], wk, wv)
        gout, _ = R.gqa_attention(q[b], K, V, s_q, sc)
        for h in range(w.heads):
            g = R.head_group(h, w.heads, w.groups)
            assert np.array_equal(o_lat[0, h], c[b][0])
            assert np.array_equal(out[0, h], c[b][0] @ wv[g].T)
            assert np.array_equal(gout[0, h], V[g, 0])


def test_zero_query_gives_mean_of_values():
    """q = 0 makes every score 0, so the output is the plain mean of the visible V rows."""
    w = workload("llama3-8b-b32-ctx8k")
    s_q = 2
    x = generate(w, s_q, batch=1, ctx_lens=[100])
    c, kr, wk, wv, qn, qr, _ = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    out, lse = R.mla_expanded_attention(c[0], kr[0], wk, wv, 0 * qn[0], 0 * qr[0], s_q, sc)
    for i in range(s_q):
        n = 100 - s_q + 1 + i
        for h in range(w.heads):
            g = R.head_group(h, w.heads, w.groups)
            assert _rel(out[i, h], (c[0][:n] @ wv[g].T).mean(axis=0)) < 1e-13
            assert abs(lse[i, h] - math.log(n)) < 1e-13


@pytest.mark.parametrize("groups", [1, 8])
def test_group_limits_mqa_and_mha(groups):
    """G = 1 is MQA (all heads share one key/value head), G = H is MHA (one key/value head
    per query head) (glossary, "Fonctionnement de la GQA"). Both paths reduce to plain
    SDPA with per-head or broadcast K/V."""
    w = workload("tiny-fp32").with_(groups=groups)
    s_q = 2
    x = generate(w, s_q, batch=1, ctx_lens=[40])
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    K, V = R.expand_latent(c[0], kr[0], wk, wv)
    assert K.shape[0] == groups
    if groups == 1:
        Kf, Vf = np.repeat(K, w.heads, 0), np.repeat(V, w.heads, 0)
    else:
        Kf, Vf = K, V
    ref = _sdpa_bottom_right(q[0], Kf, Vf, s_q, sc, False)
    out, _ = R.mla_expanded_attention(c[0], kr[0], wk, wv, qn[0], qr[0], s_q, sc)
    assert _rel(out, ref) < 1e-12
    ab = R.batch_absorb(c, kr, wk, wv, qn, qr, s_q, sc)[0][3]
    assert _rel(ab, ref) < 1e-12


def test_head_group_map_is_repeat_interleave():
    """Head h uses key/value head h // gs, which is what repeat_interleave along the head
    axis builds (glossary example)."""
    H, G = 32, 8
    idx = torch.arange(G).repeat_interleave(H // G).tolist()
    assert [R.head_group(h, H, G) for h in range(H)] == idx
    with pytest.raises(ValueError):
        R.head_group(0, 10, 4)


# -------------------------------------------------------------- printed-value pins

def test_printed_cache_sizes():
    g = json.load(open(os.path.join(GOLDEN, "cache_sizes.json")))
    a = g["llama3_8b_gqla"]
    latent = R.latent_values_per_token(a["latent"], a["rope"])
    gqa = R.kv_values_per_token(a["kv_heads"], a["head_dim"])
    assert (latent, gqa) == (576, 2048)
    assert latent / gqa == a["absorb_fraction_of_gqa"]
    # the expanded cache of the LLaMA-3-8B-shaped GQLA layer (8 groups, d_qk = d_v = 128)
    # has exactly the GQA baseline's size: "GQA-level traffic" on the per-group path
    assert R.expanded_values_per_token(8, 64 + 64, 128) == gqa
    m = g["llama31_8b_cache"]
    per_tok = m["layers"] * R.kv_values_per_token(m["kv_heads"], m["head_dim"]) * m["bytes_per_value"]
    assert per_tok == m["gqa_bytes_per_token"] == 128 * 1024
    assert per_tok * m["context"] == m["gqa_bytes_full_context"] == 16 * 2**30
    mha = m["layers"] * R.kv_values_per_token(m["query_heads"], m["head_dim"]) * m["bytes_per_value"]
    assert mha == m["mha_bytes_per_token"] and mha * m["context"] == m["mha_bytes_full_context"]


def test_printed_sdpa_gqa_example():
    """Our own rerun of the glossary's experiment (8 query heads, 2 key/value heads, 16
    tokens, 64 dims, causal) reproduces its printed shape, equality and cache counts, and
    the oracle's gqa_attention (bottom-right causal, which is the same mask for a square
    score matrix) agrees with it."""
    g = json.load(open(os.path.join(GOLDEN, "gqa_sdpa_example.json")))
    gen = torch.Generator().manual_seed(0)
    Hq, Hk, T, D = g["query_heads"], g["kv_heads"], g["tokens"], g["head_dim"]
    q = torch.randn(g["batch"], Hq, T, D, generator=gen)
    k = torch.randn(g["batch"], Hk, T, D, generator=gen)
    v = torch.randn(g["batch"], Hk, T, D, generator=gen)
    out = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    rep = Hq // Hk
    ref = F.scaled_dot_product_attention(q, k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1),
                                         is_causal=True)
    assert list(out.shape) == g["output_shape"]
    assert torch.allclose(out, ref, atol=1e-6) == g["same_as_copied_heads"]
    assert R.kv_values_per_token(Hk, D) == g["cached_values_gqa"]
    assert R.kv_values_per_token(Hq, D) == g["cached_values_mha"]
    o64, _ = R.gqa_attention(q[0].double().numpy().transpose(1, 0, 2), k[0].double().numpy(),
                             v[0].double().numpy(), T, 1.0 / math.sqrt(D))
    assert _rel(o64.transpose(1, 0, 2), out[0].double().numpy()) < 1e-5


# --------------------------------------------------------------------- invariants

def test_split_merge_identity():
    """Softmax averages over disjoint ranges, merged by their log-sum-exp, equal the
    average over the union (including empty ranges)."""
    rng = np.random.default_rng(7)
    s = rng.standard_normal(1000) * 3
    v = rng.standard_normal((1000, 40))
    o, l = R.softmax_average(s, v)
    for bounds in ([0, 1000], [0, 64, 128, 1000], [0, 0, 500, 500, 1000], [0, 1, 999, 1000],
                   sorted(set([0, 1000] + rng.integers(0, 1000, 9).tolist()))):
        mo, ml = R.attention_over_ranges(s, v, bounds)
        assert np.max(np.abs(mo - o)) < 1e-13 and abs(ml - l) < 1e-12


def test_paged_gather_and_block_shuffle():
    """Gathering through the block table returns the logical rows bit for bit, and a
    shuffled table gives bit-identical oracle outputs (the oracle works in logical order)."""
    w = workload("tiny-fp32")
    s_q = 2
    ctx = [130, 64, 1 + s_q]
    a = generate(w, s_q, batch=3, ctx_lens=ctx, shuffled=False)
    b = generate(w, s_q, batch=3, ctx_lens=ctx, shuffled=True, extra_blocks=3)
    assert not np.array_equal(a.block_table, b.block_table)
    sc = R.qk_scale(w.nope, w.rope)
    for x in (a, b):
        cache = x.f64(x.latent_cache)
        for i in range(3):
            rows = R.gather_tokens(cache, x.block_table[i], int(x.ctx_lens[i]))
            assert np.array_equal(rows[:, :w.latent], x.f64(x.c_kv_seq[i]))
            assert np.array_equal(rows[:, w.latent:], x.f64(x.k_rope_seq[i]))
    outs = []
    for x in (a, b):
        cache = x.f64(x.latent_cache)
        res = []
        for i in range(3):
            rows = R.gather_tokens(cache, x.block_table[i], int(x.ctx_lens[i]))
            res.append(R.mla_expanded_attention(rows[:, :w.latent], rows[:, w.latent:], x.f64(x.w_uk),
                                                x.f64(x.w_uv), x.f64(x.q_nope[i]), x.f64(x.q_rope[i]),
                                                s_q, sc)[0])
        outs.append(res)
    for p, q in zip(*outs):
        assert np.array_equal(p, q)


def test_expand_blocks_follow_block_table():
    """Expanding the physical blocks listed by a sequence's table row, read back in table
    order, equals expanding its logical latent rows."""
    w = workload("tiny-fp32")
    x = generate(w, 1, batch=2, ctx_lens=[150, 70], shuffled=True)
    cache = x.f64(x.latent_cache)
    wk, wv = x.f64(x.w_uk), x.f64(x.w_uv)
    for b in range(2):
        L = int(x.ctx_lens[b])
        nb = (L + 63) // 64
        Kb, Vb = R.expand_blocks(cache, x.block_table[b, :nb], wk, wv, w.latent)
        K, V = R.expand_latent(x.f64(x.c_kv_seq[b]), x.f64(x.k_rope_seq[b]), wk, wv)
        Kl = Kb.transpose(1, 0, 2, 3).reshape(w.groups, nb * 64, -1)[:, :L]
        Vl = Vb.transpose(1, 0, 2, 3).reshape(w.groups, nb * 64, -1)[:, :L]
        assert np.allclose(Kl, K, rtol=0, atol=1e-12) and np.allclose(Vl, V, rtol=0, atol=1e-12)


def test_rope_rotation_properties():
    """Rotary embedding preserves norms and <R(m) q, R(n) k> depends only on m - n."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m in (0, 5, 1000, 65535):
        assert abs(np.linalg.norm(rope_rotate(q, m)) - np.linalg.norm(q)) < 1e-12
    d = [rope_rotate(q, m) @ rope_rotate(k, m - 7) for m in (7, 100, 40000)]
    assert max(d) - min(d) < 1e-9
    assert np.allclose(rope_rotate(q, 0), q)


# ----------------------------------------------------------------- planted mistakes

def _mutant(**replace):
    """A copy of the oracle module with some functions replaced (CPU only)."""
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update(R.__dict__)
    for k, fn in replace.items():
        m.__dict__[k] = fn
    for name in ("mla_expanded_attention", "absorb_query", "absorb_attention", "out_projection",
                 "gqa_attention", "expand_latent", "batch_absorb", "batch_naive", "batch_gqa"):
        f = R.__dict__[name]
        m.__dict__[name] = types.FunctionType(f.__code__, m.__dict__, name, f.__defaults__)
    for k, fn in replace.items():
        m.__dict__[k] = fn
    return m


def _pins_pass(M, s_q=2):
    """Run the path-equivalence, SDPA and one-token pins against module M."""
    w = workload("tiny-fp32")
    x = generate(w, s_q, batch=1, ctx_lens=[48])
    c, kr, wk, wv, qn, qr, q = _f64_inputs(x)
    sc = R.qk_scale(w.nope, w.rope)
    out, _ = M.mla_expanded_attention(c[0], kr[0], wk, wv, qn[0], qr[0], s_q, sc)
    ab = M.batch_absorb(c, kr, wk, wv, qn, qr, s_q, sc)[0][3]
    K, V = R.expand_latent(c[0], kr[0], wk, wv)
    ref = _sdpa_bottom_right(q[0], K, V, s_q, sc, False)
    gq = M.batch_gqa(c, kr, wk, wv, q, s_q, sc)[0][0]
    return _rel(out, ref) < 1e-12 and _rel(ab, ref) < 1e-12 and _rel(gq, ref) < 1e-12


def test_pins_pass_on_the_oracle():
    assert _pins_pass(R)


@pytest.mark.parametrize("mistake", ["group_map", "causal_off_by_one", "no_rope_in_absorb",
                                     "transposed_value_proj"])
def test_pins_catch_planted_mistakes(mistake):
    if mistake == "group_map":
        M = _mutant(head_group=lambda h, H, G: h % G)
    elif mistake == "causal_off_by_one":
        M = _mutant(visible_tokens=lambda L, s_q, i: L - s_q + i if i else L - s_q + 1)
    elif mistake == "no_rope_in_absorb":
        def absorb_query(q_nope, q_rope, w_uk):
            qa = R.absorb_query(q_nope, q_rope, w_uk)
            qa[..., w_uk.shape[2]:] = 0.0
            return qa
        M = _mutant(absorb_query=absorb_query)
    else:
        def out_projection(o_lat, w_uv):
            H = o_lat.shape[-2]
            G, d_v, d_c = w_uv.shape
            out = np.zeros(o_lat.shape[:-1] + (d_v,))
            for h in range(H):
                wt = w_uv[R.head_group(h, H, G)].reshape(d_c, d_v).T  # wrong orientation
                out[..., h, :] = o_lat[..., h, :] @ wt.T
            return out
        M = _mutant(out_projection=out_projection)
    assert not _pins_pass(M)


# ------------------------------------------------------------------ append-path pins

def test_rope_at_worked_values():
    """RoPE closed forms (reading: half-split pairs, theta 10000). With d_R = 2 the single
    pair turns by the position itself; with d_R = 4, component 0 pairs with 2 (not 1) and
    the second pair turns at theta^(-1/2) = 1/100 of the rate."""
    t = 3.0
    assert np.allclose(R.rope_at(np.array([1.0, 0.0]), t), [math.cos(t), math.sin(t)], atol=1e-15)
    assert np.allclose(R.rope_at(np.array([1.0, 0.0, 0.0, 0.0]), t), [math.cos(t), 0, math.sin(t), 0], atol=1e-15)
    assert np.allclose(R.rope_at(np.array([0.0, 1.0, 0.0, 0.0]), t),
                       [0, math.cos(t / 100), 0, math.sin(t / 100)], atol=1e-15)


def test_rope_at_is_a_relative_rotation():
    """Position 0 is the identity, norms are kept, and <R_m q, R_n k> depends on m - n only
    (the defining property of rotary embeddings)."""
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(R.rope_at(q, 0), q)
    assert math.isclose(np.linalg.norm(R.rope_at(q, 12345)), np.linalg.norm(q), rel_tol=1e-12)
    a = R.rope_at(q, 700) @ R.rope_at(k, 300)
    b = R.rope_at(q, 400) @ k
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_append_rows_positions_and_skips():
    """New rows land at t = L - s_q + i, carry c unchanged and the key rotated to t; a
    sequence shorter than s_q writes nothing."""
    rng = np.random.default_rng(6)
    c = rng.standard_normal((3, 2, 8))
    kr = rng.standard_normal((3, 2, 4))
    rows = R.append_rows(c, kr, np.array([10, 1, 64]), 2)
    assert sorted(rows) == [(0, 8), (0, 9), (2, 62), (2, 63)]
    assert np.array_equal(rows[(2, 63)][:8], c[2, 1])
    assert np.allclose(rows[(0, 8)][8:], R.rope_at(kr[0, 0], 8))
    assert not np.allclose(rows[(0, 8)][8:], kr[0, 0])


# ------------------------------------------------------------------ output-side pins

def _out_side_inputs(seed=5, B=2, H=8, G=2, d_v=6, d_c=10, hidden=12):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, d_v)), rng.standard_normal((B, H, d_c)),
            rng.standard_normal((G, d_v, d_c)), rng.standard_normal((hidden, H * d_v)))


def test_hidden_projection_is_the_modules_linear_layer():
    """The module's last step: attention output of shape (b, H, s, head_dim) transposed to
    (b, s, H, head_dim), flattened and passed through a bias-free Linear(H*head_dim,
    hidden). Re-done here with the module's own torch operations on s = 1."""
    out, _, _, w_o = _out_side_inputs()
    t = torch.from_numpy(out)[:, :, None, :]                         # (b, H, s=1, d_v)
    flat = t.transpose(1, 2).contiguous().view(out.shape[0], 1, -1)
    lin = torch.nn.Linear(w_o.shape[1], w_o.shape[0], bias=False).double()
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w_o))
        ref = lin(flat)[:, 0].numpy()
    assert _rel(R.hidden_projection(out, w_o), ref) < 1e-14


def test_hidden_projection_head_major_order():
    """With W_O the identity (hidden = H*d_v) the projection returns feature h*d_v + v =
    value v of head h; a permutation moves exactly one value per output."""
    out, _, _, _ = _out_side_inputs(hidden=8 * 6)
    B, H, d_v = out.shape
    y = R.hidden_projection(out, np.eye(H * d_v))
    for h in range(H):
        for v in range(d_v):
            assert y[1, h * d_v + v] == out[1, h, v]
    perm = np.random.default_rng(1).permutation(H * d_v)
    y = R.hidden_projection(out, np.eye(H * d_v)[perm])
    for n in range(H * d_v):
        assert y[0, n] == out[0, perm[n] // d_v, perm[n] % d_v]


def test_fold_equals_value_then_output_projection():
    """Folding W_UV^g into W_O changes nothing: W_fold applied to the latent outputs equals
    W_O applied after W_UV^g, and a brute-force sum over heads, values and latent features
    gives the same folded weight."""
    _, o_lat, w_uv, w_o = _out_side_inputs()
    H = o_lat.shape[1]
    w_fold = R.fold_out_weight(w_o, w_uv, H)
    a = R.folded_hidden_projection(o_lat, w_fold)
    b = R.hidden_projection(R.out_projection(o_lat, w_uv), w_o)
    assert _rel(a, b) < 1e-12
    G, d_v, d_c = w_uv.shape
    for n in (0, 7):
        for h in (0, 3, 5, 7):
            for c in (0, 9):
                ref = sum(w_o[n, h * d_v + v] * w_uv[h // (H // G), v, c] for v in range(d_v))
                assert abs(w_fold[n, h * d_c + c] - ref) < 1e-12
