"""The decode calls under HIP graph capture: one step (append of the new tokens, absorb
path with its split combine, the same decode through gqla_decode_absorb_out with the combine
fused into the value projection, GQA path) captured once and replayed several times, with
eager work and synchronisations between the replays, gives the eager step's outputs bit
for bit each time (the library records no memset nodes; its kernels are deterministic)."""
import numpy as np
import pytest
import torch

from workloads import generate, queries_for, workload

from gpu_util import Run, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama3-8b-b32-ctx8k", "dsv3-b64-ctx8k"])
def test_captured_step_replays_match_eager(name):
    w = workload(name)
    x = generate(w, 2, batch=4, ctx_lens=[130, 700, 64, 2], shuffled=True, extra_blocks=2)
    run = Run(x, 3, rope_shared=True)
    G, d_gqa = run.G, run.dims
    d_abs = G.Dims(batch=run.B, num_heads=w.heads, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                   nope_dim=w.nope, v_dim=w.v, s_q=1, dtype=G.GQLA_BF16)
    qn1, qr1 = queries_for(x, 1)
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    q_nope1, q_rope1 = to_bf16(qn1), to_bf16(qr1)
    expanded = run.expand()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    c_app = torch.randn(run.B, 2, w.latent, generator=gen, device="cuda").to(torch.bfloat16)
    kr_app = torch.randn(run.B, 2, w.rope, generator=gen, device="cuda").to(torch.bfloat16)
    q_abs = torch.empty(run.B, 1, w.heads, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(run.B, 1, w.heads, w.latent, dtype=torch.float32, device="cuda")
    out_abs = torch.empty(run.B, 1, w.heads, w.v, dtype=torch.bfloat16, device="cuda")
    out_gqa = torch.empty(run.B, 2, w.heads, w.v, dtype=torch.bfloat16, device="cuda")
    lse_gqa = torch.empty(run.B, 2, w.heads, dtype=torch.float32, device="cuda")
    paged_abs = G.Paged(run.table, run.lens, run.paged.max_ctx_len, x.num_blocks, 3)

    def ws(dims, path):
        n = G.gqla_workspace_bytes(dims, path, run.table.shape[1], run.paged.max_ctx_len, x.num_blocks, 3)
        return torch.zeros(max(n // 4, 1), dtype=torch.float32, device="cuda")
    ws_abs, ws_gqa = ws(d_abs, G.GQLA_PATH_ABSORB), ws(d_gqa, G.GQLA_PATH_GQA)
    assert G.gqla_num_splits(d_abs, G.GQLA_PATH_ABSORB, run.table.shape[1], run.paged.max_ctx_len,
                             x.num_blocks, 3) > 1   # the combine is part of the captured step
    o_lat2, out_abs2 = torch.empty_like(o_lat), torch.empty_like(out_abs)
    outs = (out_abs, out_gqa, lse_gqa, o_lat, o_lat2, out_abs2)

    def step():
        G.gqla_append_tokens(d_gqa, run.paged, c_app, kr_app, 10000.0, run.w_uk, run.w_uv, run.cache, expanded)
        G.gqla_absorb_query(d_abs, q_nope1, q_rope1, run.w_uk, q_abs)
        G.gqla_decode_absorb(d_abs, paged_abs, q_abs, run.cache, ws_abs, o_lat)
        G.gqla_out_proj(d_abs, o_lat, run.w_uv, out_abs)
        G.gqla_decode_absorb_out(d_abs, paged_abs, q_abs, run.cache, run.w_uv, ws_abs, o_lat2, out_abs2)
        G.gqla_decode_gqa(d_gqa, run.paged, run.q, expanded, ws_gqa, out_gqa, lse_gqa)

    log(f"graph capture {name}")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert all(torch.isfinite(t).all() for t in ref)
    # the two absorb forms differ only in the order of the combine's sums
    assert float((o_lat2 - o_lat).abs().max()) <= 1e-5 * float(o_lat.abs().max())
    assert float((out_abs2.float() - out_abs.float()).abs().max()) <= 1e-2 * float(out_abs.float().abs().max())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        ws_abs.fill_(float("nan"))            # stale partials must not leak into a replay
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (rep, k)
        step()                                 # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
    log("  4 replays identical to the eager step")
