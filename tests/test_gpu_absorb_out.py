"""gqla_decode_absorb_out: the absorb decode and the value projection in one call (split
combine fused with W_UV^g) against the fp64 oracle and against the two-call path
(gqla_decode_absorb then gqla_out_proj), at split counts that take the fused kernel (3, 8,
16, automatic) and that do not (unsplit, more than 64 splits), on ragged and one-token
contexts, at each of its row tiles (4, 8 and 16 rows per workgroup)."""
import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from workloads import generate, workload

from gpu_util import TOL, Run, log, oracle_paths, rel_err, to_host, torch_dtype

pytestmark = pytest.mark.gpu


def _fused_and_two_call(x, splits):
    run = Run(x, splits)
    w = x.w
    dt = torch_dtype(x.dtype)
    B = run.B
    q_abs = torch.empty(B, x.s_q, w.heads, w.latent + w.rope, dtype=dt, device="cuda")
    G.gqla_absorb_query(run.dims, run.q_nope, run.q_rope, run.w_uk, q_abs)
    res = {}
    for name in ("fused", "two-call"):
        ws = run.workspace(G.GQLA_PATH_ABSORB)
        if ws is not None:
            ws.fill_(float("nan"))
        o_lat = torch.full((B, x.s_q, w.heads, w.latent), float("nan"), device="cuda")
        lse = torch.full((B, x.s_q, w.heads), float("nan"), device="cuda")
        out = torch.full((B, x.s_q, w.heads, w.v), float("nan"), dtype=dt, device="cuda")
        if name == "fused":
            G.gqla_decode_absorb_out(run.dims, run.paged, q_abs, run.cache, run.w_uv, ws, o_lat, out, lse)
        else:
            G.gqla_decode_absorb(run.dims, run.paged, q_abs, run.cache, ws, o_lat, lse)
            G.gqla_out_proj(run.dims, o_lat, run.w_uv, out)
        torch.cuda.synchronize()
        res[name] = dict(o_lat=to_host(o_lat), lse=to_host(lse), out=to_host(out))
    n = G.gqla_num_splits(run.dims, G.GQLA_PATH_ABSORB, run.table.shape[1], run.paged.max_ctx_len,
                          run.paged.num_blocks, splits)
    return n, res


CASES = [  # workload, s_q, contexts, forced splits (0 = automatic)
    ("llama3-8b-b32-ctx8k", 1, [3000, 700, 65, 1, 2500, 4096], 0),
    ("llama3-8b-b32-ctx8k", 1, [3000, 700, 65, 1, 2500, 4096], 8),
    ("llama3-8b-b32-ctx8k", 2, [129, 700, 2, 1000], 3),
    ("dsv3-b64-ctx8k", 2, [300, 65, 1000, 2], 3),
    ("dsv3-b64-ctx8k", 1, [1500, 64, 129], 16),
    ("dsv3-tp8share-ctx16k", 2, [900, 2, 513, 64, 1200], 0),
    ("dsv3-b64-ctx8k", 2, [300, 65], 1),
    ("dsv3-b64-ctx8k", 1, [6000, 4500], 90),
    ("tiny-fp32", 2, [64, 2, 130, 65], 3),
    # row tiles of the fused kernel: 4 rows above; 8 rows (128 rows per group, 16 groups);
    # 16 rows (256 rows per group)
    ("dsv3-b64-ctx8k", 2, [2, 70, 130, 200, 65, 64, 3, 150], 3),
    ("dsv3-b64-ctx8k", 1, [(37 * i) % 190 + 1 for i in range(32)], 5),
]


@pytest.mark.parametrize("name,s_q,ctx,splits", CASES)
def test_decode_absorb_out_matches_oracle_and_two_calls(name, s_q, ctx, splits):
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=ctx, shuffled=True, extra_blocks=1)
    log(f"absorb_out {name} s_q={s_q} ctx={ctx} splits={splits}")
    n, res = _fused_and_two_call(x, splits)
    ref = oracle_paths(x)
    tol = TOL[x.dtype]
    f, t = res["fused"], res["two-call"]
    worst = 0.0
    for b in ref:
        e_out = rel_err(f["out"][b], ref[b]["absorb_out"])
        e_lat = rel_err(f["o_lat"][b], ref[b]["o_lat"])
        e_lse = float(np.max(np.abs(f["lse"][b] - ref[b]["absorb_lse"])))
        worst = max(worst, e_out, e_lat)
        assert e_out <= tol and e_lat <= tol, (b, e_out, e_lat)
        assert e_lse <= tol * max(1.0, float(np.max(np.abs(ref[b]["absorb_lse"])))), (b, e_lse)
    # the two forms differ only in the order of a sum (the combine's weight total)
    d_out = rel_err(f["out"], t["out"])
    d_lat = float(np.max(np.abs(f["o_lat"] - t["o_lat"])) / np.max(np.abs(t["o_lat"])))
    log(f"  {n} splits: worst vs oracle {worst:.2e}; fused vs two calls: out {d_out:.1e}, o_lat {d_lat:.1e}")
    assert d_lat <= 1e-5 and d_out <= tol
