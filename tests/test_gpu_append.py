"""GPU parity of gqla_append_tokens (the append path).

The s_q new tokens of every sequence must land at positions L - s_q + i of the paged
latent cache as [c ; RoPE_t(k_rope)] (c bit-exact, the rotated key within one rounding
step of the oracle's fp64 rope_at), their K/V in every group must match the oracle's
expansion of that row, every other slot of both caches must stay bit-identical, and the
decode paths over the updated caches must match the oracle on the updated sequences."""
import numpy as np
import pytest
import torch

from oracle import gqla_ref as R
from workloads import f64_to_bf16_bits, generate, workload

from gpu_util import TOL, Run, expanded_to_logical, log, oracle_paths, rel_err, to_dev

pytestmark = pytest.mark.gpu

THETA = 10000.0


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy().copy()


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f64_to_bf16_bits(a) if dtype == "bf16" else a.astype(np.float32)


def _append(name, dtype, s_q, ctx, seed, bad_first=False, rope_shared=False):
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=ctx, dtype=dtype, shuffled=True, extra_blocks=2)
    if bad_first:
        x.ctx_lens[0] = s_q - 1   # metadata the append must skip
    run = Run(x, 0, rope_shared)
    expanded = run.expand()
    lat0, exp0 = _bits(run.cache), _bits(expanded)
    rng = np.random.default_rng(seed)
    B = len(ctx)
    c_new = _store(rng.standard_normal((B, s_q, w.latent)), dtype)
    kr_new = _store(rng.standard_normal((B, s_q, w.rope)), dtype)
    log(f"append {name} {dtype} s_q={s_q} ctx={list(x.ctx_lens)}")
    run.G.gqla_append_tokens(run.dims, run.paged, to_dev(c_new, dtype), to_dev(kr_new, dtype), THETA,
                             run.w_uk, run.w_uv, run.cache, expanded)
    torch.cuda.synchronize()
    return x, run, expanded, lat0, exp0, c_new, kr_new


@pytest.mark.parametrize("name,dtype,s_q,ctx", [
    ("tiny-fp32", "f32", 2, [2, 64, 65, 100]),
    ("llama3-8b-b32-ctx8k", "bf16", 2, [2, 63, 64, 65, 129, 700]),
    ("dsv3-b64-ctx8k", "bf16", 1, [1, 64, 300, 4096]),
    ("dsv3-b64-ctx8k", "bf16", 4, [5, 66, 130]),
    # several 16-token tiles, the last one ragged (22 and 18 new tokens)
    ("llama3-8b-b32-ctx8k", "bf16", 2, [2, 63, 64, 65, 129, 700, 3, 90, 191, 257, 1000]),
    ("dsv3-b64-ctx8k", "bf16", 2, [2, 64, 65, 127, 128, 129, 640, 641, 1500]),
])
@pytest.mark.parametrize("bad_first,rope_shared", [(False, False), (True, False), (False, True)])
def test_append_writes_exactly_the_new_slots(name, dtype, s_q, ctx, bad_first, rope_shared):
    x, run, expanded, lat0, exp0, c_new, kr_new = _append(name, dtype, s_q, ctx, 11, bad_first, rope_shared)
    w = x.w
    lat1, exp1 = _bits(run.cache), _bits(expanded)
    rows = R.append_rows(x.f64(c_new), x.f64(kr_new), x.ctx_lens, s_q, THETA)
    if bad_first:
        assert not any(b == 0 for b, _ in rows)
    new = np.zeros(lat1.shape[:2], dtype=bool)
    got_lat = x.f64(lat1.view(np.uint16) if dtype == "bf16" else lat1.view(np.float32))
    lay = (rope_shared, w.rope)
    K1, V1 = expanded_to_logical(x.f64(exp1.view(np.uint16) if dtype == "bf16" else exp1.view(np.float32)),
                                 x.num_blocks, w.groups, w.qk, w.v, *lay)
    lat_bits = lat1.reshape(lat1.shape[0], 64, -1)
    k_bits, _ = expanded_to_logical(exp1, x.num_blocks, w.groups, w.qk, w.v, *lay)
    worst_rope, worst_kv, kv_scale = 0.0, 0.0, 0.0
    f64w_uk, f64w_uv = x.f64(x.w_uk), x.f64(x.w_uv)
    for (b, t), row in rows.items():
        p, s = int(x.block_table[b, t // 64]), t % 64
        new[p, s] = True
        i = t - (int(x.ctx_lens[b]) - s_q)
        assert np.array_equal(lat_bits[p, s, :w.latent], c_new[b, i].view(lat_bits.dtype)), (b, t)
        ref_rope = row[w.latent:]
        step = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
        worst_rope = max(worst_rope, float(np.max(np.abs(got_lat[p, s, w.latent:] - ref_rope) /
                                                 np.maximum(np.abs(ref_rope), 1e-30))))
        assert np.all(np.abs(got_lat[p, s, w.latent:] - ref_rope) <= step * np.abs(ref_rope) + 1e-30), (b, t)
        # K's RoPE part is the cached key itself; K's nope part and V come from c alone.
        for g in range(w.groups):
            assert np.array_equal(k_bits[p, g, s, w.nope:], lat_bits[p, s, w.latent:]), (b, t, g)
        K, V = R.expand_latent(row[None, :w.latent], row[None, w.latent:], f64w_uk, f64w_uv)
        err = max(np.max(np.abs(K1[p, :, s, :w.nope] - K[:, 0, :w.nope])), np.max(np.abs(V1[p, :, s] - V[:, 0])))
        worst_kv = max(worst_kv, float(err))
        kv_scale = max(kv_scale, float(np.max(np.abs(K[:, 0, :w.nope]))), float(np.max(np.abs(V))))
    log(f"  {len(rows)} rows: rope rel {worst_rope:.2e}, K/V abs {worst_kv:.2e} (scale {kv_scale:.2f})")
    assert worst_kv <= TOL[dtype] * kv_scale
    # everything else untouched, bit for bit
    lat0r = lat0.reshape(lat1.shape[0], 64, -1)
    assert np.array_equal(lat0r[~new], lat_bits[~new])
    k0, v0 = expanded_to_logical(exp0, x.num_blocks, w.groups, w.qk, w.v, *lay)
    k1b, v1b = expanded_to_logical(exp1, x.num_blocks, w.groups, w.qk, w.v, *lay)
    for g in range(w.groups):
        assert np.array_equal(k0[:, g][~new], k1b[:, g][~new])
        assert np.array_equal(v0[:, g][~new], v1b[:, g][~new])


@pytest.mark.parametrize("name,dtype,s_q,ctx", [
    ("tiny-fp32", "f32", 2, [2, 64, 100]),
    ("llama3-8b-b32-ctx8k", "bf16", 2, [63, 65, 700]),
    ("dsv3-b64-ctx8k", "bf16", 2, [2, 129]),
])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_decode_after_append_matches_oracle(name, dtype, s_q, ctx, rope_shared):
    x, run, expanded, _, _, c_new, kr_new = _append(name, dtype, s_q, ctx, 12, rope_shared=rope_shared)
    w = x.w
    # The updated sequences, as cached (the key rotated and rounded on the GPU).
    lat = _bits(run.cache).reshape(x.num_blocks, 64, -1)
    store = np.uint16 if dtype == "bf16" else np.float32
    for b in range(len(ctx)):
        L = int(x.ctx_lens[b])
        for t in range(L - s_q, L):
            row = lat[int(x.block_table[b, t // 64]), t % 64].view(store)
            x.c_kv_seq[b][t] = row[:w.latent]
            x.k_rope_seq[b][t] = row[w.latent:]
    got_a, got_g = run.absorb(), run.gqa(expanded)
    ref = oracle_paths(x)
    for b in ref:
        ea, eg = rel_err(got_a["out"][b], ref[b]["out"]), rel_err(got_g["out"][b], ref[b]["out"])
        log(f"  seq {b}: absorb {ea:.2e} gqa {eg:.2e}")
        assert ea <= TOL[dtype] and eg <= TOL[dtype]


@pytest.mark.parametrize("name,dtype,s_q,ctx", [
    ("tiny-fp32", "f32", 2, [2, 64, 65, 100]),
    ("llama3-8b-b32-ctx8k", "bf16", 2, [2, 63, 64, 65, 129, 700, 3, 90, 191, 257, 1000]),
    ("dsv3-tp8share-ctx16k", "bf16", 2, [2, 64, 65, 127, 1500]),
])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_append_without_latent_cache_writes_the_same_expanded_cache(name, dtype, s_q, ctx, rope_shared):
    """A GQA-only deployment passes no latent cache: the expanded cache must come out bit-identical
    to the append that also writes the latent rows."""
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=ctx, dtype=dtype, shuffled=True, extra_blocks=2)
    run = Run(x, 0, rope_shared)
    expanded = run.expand()
    exp_only = expanded.clone()
    before = _bits(expanded)
    rng = np.random.default_rng(21)
    c_new = to_dev(_store(rng.standard_normal((len(ctx), s_q, w.latent)), dtype), dtype)
    kr_new = to_dev(_store(rng.standard_normal((len(ctx), s_q, w.rope)), dtype), dtype)
    log(f"append without latent {name} {dtype} s_q={s_q} rope_shared={rope_shared}")
    run.G.gqla_append_tokens(run.dims, run.paged, c_new, kr_new, THETA, run.w_uk, run.w_uv, run.cache, expanded)
    run.G.gqla_append_tokens(run.dims, run.paged, c_new, kr_new, THETA, run.w_uk, run.w_uv, None, exp_only)
    torch.cuda.synchronize()
    assert not np.array_equal(_bits(expanded), before)   # the append wrote something
    assert np.array_equal(_bits(expanded), _bits(exp_only))
    with pytest.raises(run.G.GqlaError):
        run.G.gqla_append_tokens(run.dims, run.paged, c_new, kr_new, THETA, run.w_uk, run.w_uv, None, None)


@pytest.mark.parametrize("name,dtype,s_q,ctx", [
    ("tiny-fp32", "f32", 2, [2, 64, 65, 100]),
    ("llama3-8b-b32-ctx8k", "bf16", 1, [1, 63, 64, 65, 129, 700, 3, 90, 191, 257, 1000, 8192, 4, 5, 6, 7, 8, 9]),
    ("dsv3-b64-ctx8k", "bf16", 2, [2, 64, 65, 127, 1500]),
])
def test_append_without_expanded_cache_writes_the_same_latent_cache(name, dtype, s_q, ctx):
    """The absorb path keeps no expanded cache: the latent rows must come out bit-identical to
    the append that also expands them."""
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=ctx, dtype=dtype, shuffled=True, extra_blocks=2)
    run = Run(x, 0)
    expanded = run.expand()
    lat_only = run.cache.clone()
    before = _bits(run.cache)
    rng = np.random.default_rng(22)
    c_new = to_dev(_store(rng.standard_normal((len(ctx), s_q, w.latent)), dtype), dtype)
    kr_new = to_dev(_store(rng.standard_normal((len(ctx), s_q, w.rope)), dtype), dtype)
    log(f"append without expanded cache {name} {dtype} s_q={s_q}")
    run.G.gqla_append_tokens(run.dims, run.paged, c_new, kr_new, THETA, run.w_uk, run.w_uv, run.cache, expanded)
    run.G.gqla_append_tokens(run.dims, run.paged, c_new, kr_new, THETA, run.w_uk, run.w_uv, lat_only, None)
    torch.cuda.synchronize()
    assert not np.array_equal(_bits(run.cache), before)
    assert np.array_equal(_bits(run.cache), _bits(lat_only))
