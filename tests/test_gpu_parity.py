"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same
seeded inputs. Floating point: max|gpu - ref| <= 1e-2 max|ref| (bf16 data) or
1e-5 max|ref| (fp32 data). Integer placement (expanded-cache layout, block tables):
bit-exact."""
import numpy as np
import pytest
import torch

from oracle import gqla_ref as R
from workloads import generate, workload, f64_to_bf16_bits

from gpu_util import (TOL, Run, expanded_to_logical, log, logical_to_expanded, oracle_paths, rel_err,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


def _check_paths(x, got_a, got_g, ref, tol, seqs=None, label=""):
    seqs = list(ref.keys()) if seqs is None else seqs
    for b in seqs:
        r = ref[b]
        e = dict(
            q_abs=rel_err(got_a["q_abs"][b], r["q_abs"]),
            o_lat=rel_err(got_a["o_lat"][b], r["o_lat"]),
            absorb_out=rel_err(got_a["out"][b], r["out"]),
            gqa_out=rel_err(got_g["out"][b], r["out"]),
        )
        lse_err = max(np.max(np.abs(got_a["lse"][b] - r["lse"])), np.max(np.abs(got_g["lse"][b] - r["lse"])))
        log(f"  {label} seq {b} L={int(x.ctx_lens[b])}: " + " ".join(f"{k}={v:.2e}" for k, v in e.items())
            + f" lse_abs={lse_err:.2e}")
        for k, v in e.items():
            assert v <= tol, (k, b, v)
        assert lse_err <= tol * max(1.0, float(np.max(np.abs(r["lse"])))), lse_err


@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_tiny_fp32_matches_oracle(s_q, num_splits, rope_shared):
    w = workload("tiny-fp32")
    x = generate(w, s_q, batch=4, ctx_lens=[64, s_q, 130, 65], shuffled=True)
    log(f"tiny-fp32 s_q={s_q} splits={num_splits} rope_shared={rope_shared}")
    run = Run(x, num_splits, rope_shared)
    got_a, got_g = run.absorb(), run.gqa()
    _check_paths(x, got_a, got_g, oracle_paths(x), TOL["f32"], label="tiny-fp32")


@pytest.mark.parametrize("s_q", [1, 2])
def test_tiny_dims_bf16_matches_oracle(s_q):
    w = workload("tiny-fp32").with_(dtype="bf16")
    x = generate(w, s_q, batch=5, ctx_lens=[s_q, 63, 64, 65, 300], shuffled=True, extra_blocks=2)
    log(f"tiny-bf16 s_q={s_q}")
    run = Run(x, 2)
    got_a, got_g = run.absorb(), run.gqa()
    _check_paths(x, got_a, got_g, oracle_paths(x), TOL["bf16"], label="tiny-bf16")


def _selection_weights(x, rng):
    """W_UK / W_UV rows that each pick one latent coordinate (weight exactly 1): every
    expanded value is then one exact copy of a latent value."""
    w = x.w
    wk = np.zeros((w.groups, w.nope, w.latent))
    wv = np.zeros((w.groups, w.v, w.latent))
    sel_k = rng.integers(0, w.latent, (w.groups, w.nope))
    sel_v = rng.integers(0, w.latent, (w.groups, w.v))
    for g in range(w.groups):
        wk[g, np.arange(w.nope), sel_k[g]] = 1.0
        wv[g, np.arange(w.v), sel_v[g]] = 1.0
    store = (lambda a: f64_to_bf16_bits(a)) if x.dtype == "bf16" else (lambda a: a.astype(np.float32))
    return store(wk), store(wv)


@pytest.mark.parametrize("name,dtype", [("tiny-fp32", "f32"), ("tiny-fp32", "bf16"),
                                        ("dsv3-b64-ctx8k", "bf16"), ("llama3-8b-b32-ctx8k", "bf16")])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_expand_cache_selection_weights_bit_exact(name, dtype, rope_shared):
    w = workload(name).with_(dtype=dtype)
    x = generate(w, 1, batch=3, ctx_lens=[64, 100, 3], shuffled=True, extra_blocks=1)
    x.w_uk, x.w_uv = _selection_weights(x, np.random.default_rng(5))
    log(f"expand selection {name} {dtype} rope_shared={rope_shared}")
    run = Run(x, 0, rope_shared)
    # expand all blocks but the spare one: it must stay untouched (NaN)
    used = np.unique(x.block_table[x.block_table >= 0]).astype(np.int32)
    ids = torch.from_numpy(used).cuda()
    flat = to_host(run.expand(ids))
    K, V = expanded_to_logical(flat, x.num_blocks, w.groups, w.qk, w.v, rope_shared, w.rope)
    cache = x.f64(x.latent_cache)
    Kr, Vr = R.expand_blocks(cache, used, x.f64(x.w_uk), x.f64(x.w_uv), w.latent)
    spare = sorted(set(range(x.num_blocks)) - set(used.tolist()))
    for j, p in enumerate(used):
        live = ~np.isnan(cache[p, :, 0])
        assert np.array_equal(K[p][:, live], Kr[j][:, live]), p
        assert np.array_equal(V[p][:, live], Vr[j][:, live]), p
    for p in spare:
        assert np.isnan(K[p]).all() and np.isnan(V[p]).all()


@pytest.mark.parametrize("name", ["tiny-fp32", "dsv3-b64-ctx8k", "llama3-8b-b32-ctx8k"])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_expand_cache_matches_oracle(name, rope_shared):
    w = workload(name)
    x = generate(w, 1, batch=2, ctx_lens=[128, 70], shuffled=True)
    log(f"expand parity {name} rope_shared={rope_shared}")
    run = Run(x, 0, rope_shared)
    flat = to_host(run.expand())
    K, V = expanded_to_logical(flat, x.num_blocks, w.groups, w.qk, w.v, rope_shared, w.rope)
    cache = x.f64(x.latent_cache)
    ids = np.arange(x.num_blocks)
    Kr, Vr = R.expand_blocks(cache, ids, x.f64(x.w_uk), x.f64(x.w_uv), w.latent)
    live = ~np.isnan(cache[:, :, 0])            # [NB][64]
    for g in range(w.groups):
        kg, kr = K[:, g][live], Kr[:, g][live]
        vg, vr = V[:, g][live], Vr[:, g][live]
        tol = TOL[x.dtype]
        assert rel_err(kg, kr) <= tol and rel_err(vg, vr) <= tol
        # the RoPE part is a copy: bit-exact
        assert np.array_equal(kg[:, w.nope:], kr[:, w.nope:])


def test_shuffled_block_table_is_bit_identical():
    """The same logical sequence stored under an identity and a shuffled block table
    produces bit-identical outputs on both paths."""
    w = workload("tiny-fp32").with_(dtype="bf16")
    a = generate(w, 2, batch=3, ctx_lens=[200, 64, 5], shuffled=False)
    b = generate(w, 2, batch=3, ctx_lens=[200, 64, 5], shuffled=True, extra_blocks=4)
    log("shuffle invariance tiny-bf16")
    ra, rb = Run(a, 2), Run(b, 2)
    for k in ("out", "o_lat", "lse"):
        assert np.array_equal(ra.absorb()[k], rb.absorb()[k]), k
    ga, gb = ra.gqa(), rb.gqa()
    assert np.array_equal(ga["out"], gb["out"]) and np.array_equal(ga["lse"], gb["lse"])


def test_bad_metadata_gives_nan_rows():
    """Block ids outside the pool are never read and poison only their sequence; a
    context longer than the block table allows poisons its sequence."""
    w = workload("tiny-fp32")
    x = generate(w, 1, batch=3, ctx_lens=[100, 100, 100])
    x.block_table[1, 1] = x.num_blocks + 1000   # out of range id, in the used part
    log("bad metadata tiny-fp32")
    run = Run(x, 0)
    run.lens[2] = 64 * x.block_table.shape[1] + 1  # longer than the table allows
    ga, aa = run.gqa(), run.absorb()
    for got in (ga["out"], aa["o_lat"], aa["out"]):
        assert np.isfinite(got[0]).all()
        assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
