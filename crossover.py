"""Absorb-vs-GQA crossover sweep on one GPU, and how gqla_pick_path's choice compares.

For each layer shape and s_q it times one decode step of each GQLA path on random data
(the same work bench.py counts in a step):
  absorb: gqla_absorb_query -> gqla_decode_absorb_out (decode; combine fused with W_UV^g)
  GQA:    gqla_expand_cache of the blocks holding the new tokens -> gqla_decode_gqa
and prints one JSON line per case plus a markdown table. The shapes are the DeepSeek-V3
attention layer and its 1/R tensor-parallel head shares (H = 128/R query heads in
G = 16/R groups, R = 1, 2, 4, 8) and the LLaMA-3-8B layer converted to GQLA.

The GQA path's expanded cache is in the layout that stores the RoPE key once per block
unless --gqa-layout per-group is given.

Usage: python crossover.py [--batch 64] [--ctx 8192] [--sq 1,2,4] [--reps 10]
                            [--gqa-layout shared-rope|per-group] [--out FILE.md]
"""
import argparse
import json
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from decode_attention_02_amd import _lib as L  # noqa: E402

# name: (heads, groups, nope_dim, v_dim)
SHAPES = {
    "dsv3 (R=1)": (128, 16, 128, 128),
    "dsv3 (R=2)": (64, 8, 128, 128),
    "dsv3 (R=4)": (32, 4, 128, 128),
    "dsv3 (R=8)": (16, 2, 128, 128),
    "llama3-8b": (32, 8, 64, 128),
}
LATENT, ROPE = 512, 64


def _bf16(shape, scale, gen):
    return (torch.randn(shape, device="cuda", generator=gen) * scale).to(torch.bfloat16)


def _median_us(fn, reps):
    for _ in range(3):
        fn()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def run_case(name, s_q, batch, ctx, reps, gen, rope_shared=1):
    H, Gr, dn, dv = SHAPES[name]
    nbs = (ctx + 63) // 64
    nb = batch * nbs
    d = L.Dims(batch=batch, num_heads=H, num_groups=Gr, latent_rank=LATENT, rope_dim=ROPE, nope_dim=dn,
               v_dim=dv, s_q=s_q, rope_shared=rope_shared)
    table = torch.arange(nb, dtype=torch.int32, device="cuda").reshape(batch, nbs)
    lens = torch.full((batch,), ctx, dtype=torch.int32, device="cuda")
    paged = L.Paged(table, lens, ctx, nb)
    latent = _bf16((nb, 64, LATENT + ROPE), 1.0, gen)
    w_uk = _bf16((Gr, dn, LATENT), LATENT ** -0.5, gen)
    w_uv = _bf16((Gr, dv, LATENT), LATENT ** -0.5, gen)
    q_nope = _bf16((batch, s_q, H, dn), 1.0, gen)
    q_rope = _bf16((batch, s_q, H, ROPE), 1.0, gen)
    q = torch.cat([q_nope, q_rope], dim=-1).contiguous()

    def ws(path):
        n = L.gqla_workspace_bytes(d, path, nbs, ctx, nb)
        return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None

    q_abs = torch.empty(batch, s_q, H, LATENT + ROPE, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(batch, s_q, H, LATENT, dtype=torch.float32, device="cuda")
    out = torch.empty(batch, s_q, H, dv, dtype=torch.bfloat16, device="cuda")
    ws_a, ws_g = ws(L.GQLA_PATH_ABSORB), ws(L.GQLA_PATH_GQA)

    def absorb():
        L.gqla_absorb_query(d, q_nope, q_rope, w_uk, q_abs)
        L.gqla_decode_absorb_out(d, paged, q_abs, latent, w_uv, ws_a, o_lat, out)

    t_abs = _median_us(absorb, reps)
    expanded = torch.empty(nb * 64 * L.gqla_cache_bytes_per_token(d, L.GQLA_PATH_GQA) // 2,
                           dtype=torch.bfloat16, device="cuda")
    L.gqla_expand_cache(d, latent, w_uk, w_uv, torch.arange(nb, dtype=torch.int32, device="cuda"), nb, expanded)
    first_new = (ctx - s_q) // 64
    tail = table[:, first_new:nbs].reshape(-1).contiguous()

    def gqa():
        L.gqla_expand_cache(d, latent, w_uk, w_uv, tail, tail.numel(), expanded)
        L.gqla_decode_gqa(d, paged, q, expanded, ws_g, out)

    t_gqa = _median_us(gqa, reps)
    del expanded, latent
    torch.cuda.empty_cache()
    path, est = L.gqla_pick_path(d, batch * ctx, ctx)
    faster = L.GQLA_PATH_GQA if t_gqa < t_abs else L.GQLA_PATH_ABSORB
    return {"shape": name, "heads": H, "groups": Gr, "s_q": s_q, "batch": batch, "ctx": ctx,
            "gqa_layout": "shared-rope" if rope_shared else "per-group",
            "absorb_us": t_abs, "gqa_us": t_gqa, "faster": ["absorb", "gqa"][faster],
            "gqa_over_absorb": t_abs / t_gqa - 1.0,
            "picked": ["absorb", "gqa"][path], "est_absorb_us": est[0], "est_gqa_us": est[1],
            "picked_cost": (t_abs if path == L.GQLA_PATH_ABSORB else t_gqa) / min(t_abs, t_gqa) - 1.0}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--sq", default="1,2,4")
    ap.add_argument("--shapes", default=",".join(SHAPES))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--gqa-layout", choices=("shared-rope", "per-group"), default="shared-rope")
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    rows = []
    for name in a.shapes.split(","):
        for s_q in (int(v) for v in a.sq.split(",")):
            r = run_case(name, s_q, a.batch, a.ctx, a.reps, gen, int(a.gqa_layout == "shared-rope"))
            rows.append(r)
            print(json.dumps(r), flush=True)
    lines = ["| shape | H | G | s_q | absorb us | GQA us | faster | GQA gain | picked | est absorb / GQA us | picked vs best |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['shape']} | {r['heads']} | {r['groups']} | {r['s_q']} | {r['absorb_us']:.1f} | "
                     f"{r['gqa_us']:.1f} | {r['faster']} | {r['gqa_over_absorb'] * 100:+.1f}% | {r['picked']} | "
                     f"{r['est_absorb_us']:.0f} / {r['est_gqa_us']:.0f} | {r['picked_cost'] * 100:+.1f}% |")
    table = "\n".join(lines)
    print(table)
    if a.out:
        with open(a.out, "w") as f:
            f.write(table + "\n")
    return rows


if __name__ == "__main__":
    sys.exit(0 if main() else 1)
