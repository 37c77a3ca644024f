"""gqla_decode_absorb_noalloc (the absorb decode with its split partials in the library's
fixed scratch array, for callers that cannot allocate) against gqla_decode_absorb with a
caller workspace: two calls in a row on the same GPU, the second with a smaller input (so
the scratch still holds the first call's partials), then a plan too large for the scratch.
The same kernels run on both sides, so the outputs must be bit-identical."""
import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from workloads import generate, workload

from gpu_util import Run, log

pytestmark = pytest.mark.gpu


def _both(x, splits):
    run = Run(x, splits)
    B, w = run.B, x.w
    q_abs = torch.empty(B, x.s_q, w.heads, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    G.gqla_absorb_query(run.dims, run.q_nope, run.q_rope, run.w_uk, q_abs)
    n_split = G.gqla_num_splits(run.dims, G.GQLA_PATH_ABSORB, run.table.shape[1], run.paged.max_ctx_len,
                                run.paged.num_blocks, splits)
    ws = run.workspace(G.GQLA_PATH_ABSORB)
    if ws is not None:
        ws.fill_(float("nan"))   # a slot the decode reads but did not write would show
    res = {}
    for name in ("workspace", "noalloc"):
        o_lat = torch.full((B, x.s_q, w.heads, w.latent), float("nan"), device="cuda")
        lse = torch.full((B, x.s_q, w.heads), float("nan"), device="cuda")
        if name == "workspace":
            G.gqla_decode_absorb(run.dims, run.paged, q_abs, run.cache, ws, o_lat, lse)
        else:
            G.gqla_decode_absorb_noalloc(run.dims, run.paged, q_abs, run.cache, o_lat, lse)
        torch.cuda.synchronize()
        res[name] = (o_lat.cpu().numpy(), lse.cpu().numpy())
    return n_split, res


def test_noalloc_absorb_decode_equals_the_workspace_entry_point():
    # call 1: the larger input and plan (DeepSeek-V3 heads, 4 ragged sequences at s_q = 2, 5 splits:
    # 10.5 MB of partials)
    x1 = generate(workload("dsv3-b64-ctx8k"), 2, batch=4, ctx_lens=[3000, 700, 65, 2500], shuffled=True,
                  extra_blocks=2, seed=41)
    # call 2: a smaller one (LLaMA-3-8B heads, 3 sequences at s_q = 1, 3 splits: 0.6 MB): its
    # partials land where call 1's still are
    x2 = generate(workload("llama3-8b-b32-ctx8k"), 1, batch=3, ctx_lens=[300, 1, 1000], shuffled=True, seed=42)
    sizes = []
    for label, x, splits in (("call 1", x1, 5), ("call 2", x2, 3)):
        log(f"noalloc {label}: {x.w.name} s_q={x.s_q} ctx={list(x.ctx_lens)} splits={splits}")
        n_split, res = _both(x, splits)
        assert n_split == splits
        d = Run(x, splits).dims
        need = G.gqla_workspace_bytes(d, G.GQLA_PATH_ABSORB, x.block_table.shape[1], int(x.ctx_lens.max()),
                                      x.num_blocks, splits)
        sizes.append(need)
        (o_ws, l_ws), (o_na, l_na) = res["workspace"], res["noalloc"]
        assert np.isfinite(o_ws).all() and np.isfinite(l_ws).all()
        assert np.array_equal(o_ws.view(np.uint32), o_na.view(np.uint32)), label
        assert np.array_equal(l_ws.view(np.uint32), l_na.view(np.uint32)), label
        log(f"  {label}: {need} scratch bytes, o_lat and lse bit-identical")
    assert 0 < sizes[1] < sizes[0] <= G.NOALLOC_SCRATCH_BYTES


def test_noalloc_unsplit_plan_uses_no_scratch():
    x = generate(workload("dsv3-b64-ctx8k"), 1, batch=2, ctx_lens=[130, 64], shuffled=True, seed=43)
    n_split, res = _both(x, 1)
    assert n_split == 1
    assert np.array_equal(res["workspace"][0].view(np.uint32), res["noalloc"][0].view(np.uint32))


def test_noalloc_rejects_a_plan_larger_than_its_scratch():
    # 8 sequences x 2 rows x 128 heads x 64 splits x 513 floats = 269 MB > 64 MiB; the check
    # runs on the host before anything is launched
    w = workload("dsv3-b64-ctx8k")
    d = G.Dims(batch=8, num_heads=128, num_groups=16, latent_rank=512, rope_dim=64, nope_dim=128, v_dim=128, s_q=2)
    table = torch.zeros(8, 1024, dtype=torch.int32, device="cuda")
    lens = torch.full((8,), 65536, dtype=torch.int32, device="cuda")
    paged = G.Paged(table, lens, 65536, 8192, 64)
    assert G.gqla_workspace_bytes(d, G.GQLA_PATH_ABSORB, 1024, 65536, 8192, 64) > G.NOALLOC_SCRATCH_BYTES
    q_abs = torch.zeros(8, 2, 128, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros(1, 64, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.zeros(8, 2, 128, w.latent, device="cuda")
    with pytest.raises(G.GqlaError) as e:
        G.gqla_decode_absorb_noalloc(d, paged, q_abs, cache, o_lat)
    assert e.value.status == -3 and "scratch" in str(e.value)   # GQLA_ERR_WORKSPACE
    log(f"  rejected: {e.value}")
