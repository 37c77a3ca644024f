"""Online-softmax rescaling on the GPU kernels. Every token's latent row and RoPE key are
scaled by a power of two that rises along the context (1/4, 1, 4 over three equal parts;
exact in bf16), so later blocks hold scores far above the earlier maxima: the
kernels' running reference is raised and their accumulators rescaled mid-sequence (the
test first checks, on the oracle's scores, that a block maximum exceeds every earlier one
by more than 2^8, the kernels' rescale threshold). Both paths against the oracle."""
import dataclasses

import numpy as np
import pytest

from oracle import gqla_ref as R
from workloads import f64_to_bf16_bits, generate, workload

from gpu_util import TOL, Run, log, oracle_paths, rel_err

pytestmark = pytest.mark.gpu


def _ramped(x):
    w = x.w
    lat = x.f64(x.latent_cache)
    c_seq, kr_seq = [], []
    for b, L in enumerate(x.ctx_lens):
        t = np.arange(int(L))
        g = 2.0 ** (2 * np.floor(3 * t / L) - 2)
        c = x.f64(x.c_kv_seq[b]) * g[:, None]
        kr = x.f64(x.k_rope_seq[b]) * g[:, None]
        blk, slot = x.block_table[b][t // R.BLOCK], t % R.BLOCK
        lat[blk, slot, :w.latent] = c
        lat[blk, slot, w.latent:] = kr
        c_seq.append(f64_to_bf16_bits(c))
        kr_seq.append(f64_to_bf16_bits(kr))
    return dataclasses.replace(x, latent_cache=f64_to_bf16_bits(lat), c_kv_seq=c_seq, k_rope_seq=kr_seq)


def _max_jump_log2(x, b):
    """Largest rise of a 64-token block's score maximum over all earlier blocks (log2 units),
    over the heads and rows of sequence b, from the oracle's absorbed queries."""
    w = x.w
    q_abs = R.absorb_query(x.f64(x.q_nope[b]), x.f64(x.q_rope[b]), x.f64(x.w_uk))   # [s_q][H][576]
    keys = np.concatenate([x.f64(x.c_kv_seq[b]), x.f64(x.k_rope_seq[b])], axis=-1)
    s = np.einsum("ihd,td->iht", q_abs, keys) * R.qk_scale(w.nope, w.rope) / np.log(2.0)
    L = keys.shape[0]
    best = 0.0
    for i in range(x.s_q):
        n = L - x.s_q + 1 + i
        blocks = [s[i, :, k:min(k + R.BLOCK, n)].max(axis=-1) for k in range(0, n, R.BLOCK)]
        run = blocks[0]
        for m in blocks[1:]:
            best = max(best, float(np.max(m - run)))
            run = np.maximum(run, m)
    return best


@pytest.mark.parametrize("name,s_q", [("llama3-8b-b32-ctx8k", 1), ("dsv3-b64-ctx8k", 2), ("dsv3-tp8share-ctx16k", 1)])
def test_rising_scores_match_oracle(name, s_q):
    w = workload(name)
    x = _ramped(generate(w, s_q, batch=3, ctx_lens=[700, 1000, 333], shuffled=True, extra_blocks=2))
    jumps = [_max_jump_log2(x, b) for b in range(3)]
    assert min(jumps) > 8.0, jumps
    log(f"rising scores {name} s_q={s_q}: largest block-max rise {min(jumps):.1f}..{max(jumps):.1f} (log2)")
    run = Run(x, 0, rope_shared=True)
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
