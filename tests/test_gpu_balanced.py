"""GPU parity of the GQA decode's length-balanced split plan (ragged batches whose
sequences x groups do not cover the CUs): runs that end one sequence and start the next,
a one-block sequence inside a run, runs at the 8-block minimum, and the empty slots of
short sequences. The workspace is NaN-filled first, so a partial slot that no workgroup
writes would poison its row. Each case prints its name before it touches the GPU."""
import numpy as np
import pytest
import torch

from workloads import generate, workload

from gpu_util import TOL, Run, log, oracle_paths, rel_err, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # 16 groups: 16 runs of 10 blocks over 149 blocks
    ("dsv3-b64-ctx8k", 2, [2, 1000, 2500, 4100, 1700]),
    # 8 groups: 32 runs of 8 blocks, one-token and one-block sequences between long ones
    ("llama3-8b-b32-ctx8k", 1, [3000, 64, 65, 5000, 1, 2047]),
    # 2 groups: 128 runs at the 8-block minimum, most of them past the last block
    ("dsv3-tp8share-ctx16k", 2, [9000, 2, 3000]),
    # two MFMA row tiles (32 query rows per group) at d_qk = 192 and 128
    ("dsv3-b64-ctx8k", 4, [900, 3000, 40, 2000]),
    ("llama3-8b-b32-ctx8k", 8, [1500, 8, 4000]),
]


def _decode(run, table=None):
    G, x, w = run.G, run.x, run.x.w
    n = G.gqla_workspace_bytes(run.dims, G.GQLA_PATH_GQA, run.table.shape[1], run.paged.max_ctx_len,
                               run.paged.num_blocks, run.paged.num_splits)
    assert n > 0, "the plan should split"
    ws = torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((run.B, x.s_q, w.heads, w.v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((run.B, x.s_q, w.heads), float("nan"), device="cuda")
    paged = run.paged if table is None else G.Paged(table, run.lens, run.paged.max_ctx_len, run.paged.num_blocks, 0)
    G.gqla_decode_gqa(run.dims, paged, run.q, run.expand(), ws, out, lse)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("name,s_q,ctx", CASES)
@pytest.mark.parametrize("rope_shared", [False, True])
def test_balanced_plan_matches_oracle(name, s_q, ctx, rope_shared):
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=[max(c, s_q) for c in ctx], shuffled=True, extra_blocks=3)
    run = Run(x, 0, rope_shared)
    G = run.G
    n = G.gqla_num_splits(run.dims, G.GQLA_PATH_GQA, run.table.shape[1], run.paged.max_ctx_len, x.num_blocks)
    log(f"balanced gqa {name} s_q={s_q} ctx={list(x.ctx_lens)} rope_shared={rope_shared} slots={n}")
    out, lse = _decode(run)
    ref = oracle_paths(x)
    for b in ref:
        e = rel_err(out[b], ref[b]["out"])
        le = float(np.max(np.abs(lse[b] - ref[b]["lse"])))
        log(f"  seq {b} L={int(x.ctx_lens[b])}: out {e:.2e} lse_abs {le:.2e}")
        assert e <= TOL["bf16"] and le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(ref[b]["lse"]))))


def test_balanced_plan_out_of_pool_id_poisons_only_its_sequence():
    w = workload("dsv3-b64-ctx8k")
    x = generate(w, 2, batch=3, ctx_lens=[2500, 3000, 1200], shuffled=True, extra_blocks=3)
    run = Run(x, 0, True)
    ref = oracle_paths(x)
    table = run.table.clone()
    table[1, 5] = x.num_blocks + 7
    log("balanced gqa: out-of-pool id in sequence 1 of 3")
    out, lse = _decode(run, table)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    for b in (0, 2):
        e = rel_err(out[b], ref[b]["out"])
        log(f"  seq {b}: out {e:.2e}")
        assert e <= TOL["bf16"]


@pytest.mark.parametrize("rope_shared", [False, True])
def test_balanced_plan_many_short_sequences(rope_shared):
    """200 sequences of one group (16 heads, s_q = 2: 32 rows, two row tiles): the plan's
    prefix sum runs over all four of each lane's sequences, and most 8-block runs walk several
    one- to four-block sequences in turn; two long sequences make the context split."""
    w = workload("dsv3-tp8share-ctx16k", groups=1)
    rng = np.random.default_rng(7)
    ctx = [int(c) for c in rng.integers(2, 220, size=200)]
    ctx[7], ctx[150] = 3000, 2500
    x = generate(w, 2, batch=len(ctx), ctx_lens=ctx, shuffled=True, extra_blocks=3)
    run = Run(x, 0, rope_shared)
    G = run.G
    n = G.gqla_num_splits(run.dims, G.GQLA_PATH_GQA, run.table.shape[1], run.paged.max_ctx_len, x.num_blocks)
    log(f"balanced gqa: 200 sequences, one group, rope_shared={rope_shared}, slots={n}")
    out, lse = _decode(run)
    ref = oracle_paths(x)
    worst = 0.0
    for b in ref:
        e = rel_err(out[b], ref[b]["out"])
        le = float(np.max(np.abs(lse[b] - ref[b]["lse"])))
        worst = max(worst, e)
        assert e <= TOL["bf16"] and le <= TOL["bf16"] * max(1.0, float(np.max(np.abs(ref[b]["lse"])))), (b, e, le)
    log(f"  worst out {worst:.2e} over {len(ref)} sequences")
