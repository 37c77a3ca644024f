"""GPU parity of the MFMA kernels at the production head shapes (bf16): ragged and
one-token contexts, several split counts, shuffled block tables. Each case prints its
name before it touches the GPU."""
import numpy as np
import pytest
import torch

from oracle import gqla_ref as R
from workloads import generate, workload

from gpu_util import (TOL, Run, expanded_to_logical, log, logical_to_expanded, oracle_paths, rel_err,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu

# gs * s_q = 4, 8, 8, 16, 16 rows per group; s_q = 4 at gs = 8 and s_q = 8 at gs = 4 give
# 32 rows, i.e. two MFMA row tiles (the d_qk = 192 one with half-block load units).
SHAPES = [("llama3-8b-b32-ctx8k", 1), ("llama3-8b-b32-ctx8k", 2), ("dsv3-b64-ctx8k", 1),
          ("dsv3-b64-ctx8k", 2), ("dsv3-tp8share-ctx16k", 2), ("dsv3-b64-ctx8k", 4),
          ("llama3-8b-b32-ctx8k", 8)]


def _ctx(s_q):
    return [s_q, 63, 64, 65, 129, 700]


@pytest.mark.parametrize("name,s_q", SHAPES)
@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_gqa_decode_matches_oracle(name, s_q, num_splits, rope_shared):
    w = workload(name)
    x = generate(w, s_q, batch=6, ctx_lens=_ctx(s_q), shuffled=True, extra_blocks=3)
    log(f"gqa {name} s_q={s_q} splits={num_splits} rope_shared={rope_shared}")
    run = Run(x, num_splits, rope_shared)
    got = run.gqa()
    ref = oracle_paths(x)
    for b in ref:
        e = rel_err(got["out"][b], ref[b]["out"])
        le = float(np.max(np.abs(got["lse"][b] - ref[b]["lse"])))
        log(f"  seq {b} L={int(x.ctx_lens[b])}: out {e:.2e} lse_abs {le:.2e}")
        assert e <= TOL["bf16"] and le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(ref[b]["lse"]))))


@pytest.mark.parametrize("name,s_q", [("dsv3-b64-ctx8k", 2), ("llama3-8b-b32-ctx8k", 2)])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_gqa_decode_on_oracle_expanded_cache(name, s_q, rope_shared):
    """Decode over an expanded cache built by the oracle (rounded to bf16), so the decode
    kernel is checked on its own."""
    from workloads import f64_to_bf16_bits
    w = workload(name)
    x = generate(w, s_q, batch=3, ctx_lens=[s_q, 200, 64], shuffled=True)
    cache = x.f64(x.latent_cache)
    K, V = R.expand_blocks(np.nan_to_num(cache), np.arange(x.num_blocks), x.f64(x.w_uk), x.f64(x.w_uv), w.latent)
    flat = f64_to_bf16_bits(logical_to_expanded(K, V, rope_shared, w.rope))
    log(f"gqa-on-oracle-cache {name} s_q={s_q} rope_shared={rope_shared}")
    run = Run(x, 0, rope_shared)
    got = run.gqa(expanded=to_dev(flat, "bf16"))
    ref = oracle_paths(x)
    for b in ref:
        assert rel_err(got["out"][b], ref[b]["out"]) <= TOL["bf16"]


def test_gqa_one_token_context_is_value_row():
    """A one-token context returns that token's expanded value row: bf16 in, bf16 out,
    so the GPU output equals the expanded cache entry bit for bit."""
    w = workload("dsv3-b64-ctx8k")
    x = generate(w, 1, batch=2, ctx_lens=[1, 1], shuffled=True)
    log("gqa one-token")
    run = Run(x)
    expanded = run.expand()
    got = run.gqa(expanded)
    _, V = expanded_to_logical(to_host(expanded), x.num_blocks, w.groups, w.qk, w.v)
    for b in range(2):
        blk = x.block_table[b, 0]
        for h in range(w.heads):
            g = h // w.group_size
            assert np.array_equal(got["out"][b, 0, h], V[blk, g, 0]), (b, h)


@pytest.mark.parametrize("name,s_q", SHAPES)
@pytest.mark.parametrize("rope_shared", [False, True])
def test_paths_agree_on_gpu(name, s_q, rope_shared):
    w = workload(name)
    x = generate(w, s_q, batch=3, ctx_lens=[s_q, 333, 1000], shuffled=True)
    log(f"absorb-vs-gqa {name} s_q={s_q} rope_shared={rope_shared}")
    run = Run(x, 0, rope_shared)
    a, g = run.absorb()["out"], run.gqa()["out"]
    for b in range(3):
        assert rel_err(a[b], g[b]) <= TOL["bf16"]


ABSORB_SHAPES = [("llama3-8b-b32-ctx8k", 1), ("llama3-8b-b32-ctx8k", 2), ("dsv3-b64-ctx8k", 1),
                 ("dsv3-b64-ctx8k", 2), ("dsv3-tp8share-ctx16k", 1), ("dsv3-tp8share-ctx16k", 2),
                 ("dsv3-b64-ctx8k", 4)]


@pytest.mark.parametrize("name,s_q", ABSORB_SHAPES)
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_absorb_path_matches_oracle(name, s_q, num_splits):
    w = workload(name)
    x = generate(w, s_q, batch=6, ctx_lens=_ctx(s_q), shuffled=True, extra_blocks=3)
    log(f"absorb {name} s_q={s_q} splits={num_splits}")
    run = Run(x, num_splits)
    got = run.absorb()
    ref = oracle_paths(x)
    for b in ref:
        r = ref[b]
        e = dict(q_abs=rel_err(got["q_abs"][b], r["q_abs"]), o_lat=rel_err(got["o_lat"][b], r["o_lat"]),
                 out=rel_err(got["out"][b], r["out"]))
        le = float(np.max(np.abs(got["lse"][b] - r["lse"])))
        log(f"  seq {b} L={int(x.ctx_lens[b])}: " + " ".join(f"{k} {v:.2e}" for k, v in e.items()) + f" lse_abs {le:.2e}")
        for k, v in e.items():
            assert v <= TOL["bf16"], (k, v)
        assert le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(r["lse"]))))


@pytest.mark.parametrize("name,s_q,rope_shared", [("llama3-8b-b32-ctx8k", 1, True), ("dsv3-b64-ctx8k", 2, False)])
def test_many_splits_match_oracle(name, s_q, rope_shared):
    """16 one-block splits, so the split combine merges more than 8 partials per row (its
    general loop rather than the all-loads-at-once form), on both paths."""
    w = workload(name)
    x = generate(w, s_q, batch=3, ctx_lens=[s_q, 700, 1000], shuffled=True, extra_blocks=2)
    run = Run(x, 16, rope_shared)
    G = run.G
    for path in (G.GQLA_PATH_ABSORB, G.GQLA_PATH_GQA):
        assert G.gqla_num_splits(run.dims, path, run.table.shape[1], run.paged.max_ctx_len,
                                 x.num_blocks, 16) == 16
    log(f"many splits {name} s_q={s_q} rope_shared={rope_shared}")
    ga, gg = run.absorb(), run.gqa()
    ref = oracle_paths(x)
    for b in ref:
        r = ref[b]
        e = dict(o_lat=rel_err(ga["o_lat"][b], r["o_lat"]), absorb=rel_err(ga["out"][b], r["out"]),
                 gqa=rel_err(gg["out"][b], r["out"]))
        le = max(float(np.max(np.abs(ga["lse"][b] - r["lse"]))), float(np.max(np.abs(gg["lse"][b] - r["lse"]))))
        log(f"  seq {b} L={int(x.ctx_lens[b])}: " + " ".join(f"{k} {v:.2e}" for k, v in e.items()) + f" lse_abs {le:.2e}")
        for k, v in e.items():
            assert v <= TOL["bf16"], (k, v)
        assert le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(r["lse"]))))


def test_absorb_one_token_context_is_latent_row():
    """With one visible token the absorb decode returns that token's latent row exactly
    (fp32 o_lat of a bf16 value)."""
    w = workload("dsv3-b64-ctx8k")
    x = generate(w, 2, batch=2, ctx_lens=[2, 2], shuffled=True)
    log("absorb one-token")
    got = Run(x).absorb()
    for b in range(2):
        c0 = x.f64(x.c_kv_seq[b][0])
        for h in range(w.heads):
            assert np.array_equal(got["o_lat"][b, 0, h], c0), (b, h)


@pytest.mark.parametrize("heads,groups,s_q", [(24, 3, 2), (8, 1, 2), (8, 1, 1), (48, 6, 1)])
@pytest.mark.parametrize("rope_shared", [False, True])
def test_gqa_decode_group_counts_match_oracle(heads, groups, s_q, rope_shared):
    """Even group counts are served two groups per workgroup with the shared RoPE key, odd
    ones (3, and MQA's single group) one per workgroup: both forms against the oracle."""
    w = workload("dsv3-b64-ctx8k", heads=heads, groups=groups)
    x = generate(w, s_q, batch=5, ctx_lens=[s_q, 64, 65, 700, 1500], shuffled=True, extra_blocks=2)
    log(f"gqa groups={groups} heads={heads} s_q={s_q} rope_shared={rope_shared}")
    got = Run(x, 0, rope_shared).gqa()
    ref = oracle_paths(x)
    for b in ref:
        e = rel_err(got["out"][b], ref[b]["out"])
        le = float(np.max(np.abs(got["lse"][b] - ref[b]["lse"])))
        log(f"  seq {b} L={int(x.ctx_lens[b])}: out {e:.2e} lse_abs {le:.2e}")
        assert e <= TOL["bf16"] and le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(ref[b]["lse"]))))
