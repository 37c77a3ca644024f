"""Per-path decode throughput on every workload, one GPU.

For each workload and query-row count it times, on random data of the workload's shape
(batch, context lengths, paging), the two GQLA decode paths as a serving step runs them:
  absorb: gqla_absorb_query -> gqla_decode_absorb_out (decode; split combine fused with W_UV^g)
  GQA:    gqla_decode_gqa (+ split combine) over an expanded cache that is already resident
and, separately, the per-token cost of the append path (gqla_append_tokens of the s_q new
tokens of every sequence, latent rows + RoPE + their expansion into the groups) and the
output side after the heads (W_O, or W_O with W_UV^g folded in for the absorb path).
Every timed call is preceded by an untimed read of 1 GiB, so the 256 MiB last-level cache
holds none of the cache being read (a read, not a write: the write-back of a dirty flush
buffer would land inside the timed call); the median and the best of the timed calls are
reported with KV bytes/s and the fraction of MI355X's 8 TB/s HBM and 2.5 PFLOP/s dense
bf16 MFMA peaks that they reach.

The inputs are Gaussian (latent, RoPE keys, queries ~ N(0, 1), weights ~ N(0, 1/sqrt(d_c)))
generated on the device with a seeded generator; the expanded cache is filled the same way
rather than computed from the latent (its values do not change the work). Context lengths
and block tables follow the workload: fixed or uniform lengths, identity or permuted tables.
The one-eighth head share at batch 10240 fills about 190 GiB with either cache, so its two
paths run one after the other, each with only its own cache resident.

Usage: python path_sweep.py [--workloads a,b] [--reps 10] [--out FILE.md]
"""
import argparse
import json
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from decode_attention_02_amd import _lib as L  # noqa: E402

HBM_PEAK = 8.0e12
MFMA_PEAK = 2.5e15
FLUSH_BYTES = 1 << 30

# workload: (absorb s_q list, GQA s_q list); shapes from the workload table
CASES = {
    "tiny-fp32": ((1, 2), (1, 2)),
    "llama3-8b-b32-ctx8k": ((1, 2), (1, 2)),
    "dsv3-b64-ctx8k": ((1, 2), (1, 2)),
    "dsv3-b8-ctx32k-64k": ((2,), (2,)),
    "dsv3-tp8share-ctx16k": ((1, 2), (2,)),
}


def _time(fn, reps, flush):
    for _ in range(2):
        fn()
    ts = []
    sink = torch.zeros((), device="cuda")
    for _ in range(reps):
        sink += flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def _fill(t, gen, scale=1.0, chunk=1 << 30):
    flat = t.view(-1)
    for lo in range(0, flat.numel(), chunk):
        hi = min(flat.numel(), lo + chunk)
        flat[lo:hi] = (torch.randn(hi - lo, generator=gen, device="cuda") * scale).to(t.dtype)


def _graph_time(fn, reps, flush):
    """Median and best of `fn` captured once in a HIP graph and replayed (the same flush
    before every replay): the path's time without the host launch gaps between its kernels."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    t = _time(g.replay, reps, flush)
    del g
    return t


def run_workload(name, reps, gen, flush, rope_shared=1, graph=False, block_table="workload"):
    from workloads import workload
    w = workload(name)
    B = w.batch
    rng = np.random.default_rng(w.seed)
    lo, hi = w.ctx
    lens_h = np.full(B, lo, dtype=np.int64) if lo == hi else rng.integers(lo, hi + 1, size=B)
    nbs = (int(lens_h.max()) + 63) // 64
    nblk = (lens_h + 63) // 64
    NB = int(nblk.sum())
    if (w.shuffled and block_table == "workload") or block_table == "shuffled":
        phys = rng.permutation(NB).astype(np.int32)
    else:
        phys = np.arange(NB, dtype=np.int32)
    table_h = np.full((B, nbs), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table_h[b, :nblk[b]] = phys[o:o + nblk[b]]
        o += nblk[b]
    table = torch.from_numpy(table_h).cuda()
    lens = torch.from_numpy(lens_h.astype(np.int32)).cuda()
    max_ctx = int(lens_h.max())
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    code = L.GQLA_F32 if w.dtype == "f32" else L.GQLA_BF16
    elt = 4 if w.dtype == "f32" else 2
    dq = w.latent + w.rope
    w_uk = torch.empty(w.groups, w.nope, w.latent, dtype=dt, device="cuda")
    w_uv = torch.empty(w.groups, w.v, w.latent, dtype=dt, device="cuda")
    _fill(w_uk, gen, w.latent ** -0.5)
    _fill(w_uv, gen, w.latent ** -0.5)
    ctx = lens_h.astype(np.float64)
    absorb_sq, gqa_sq = CASES[name]
    rows = []

    def vis(s):
        return float(sum(sum(Lb - s + 1 + i for i in range(s)) for Lb in ctx))

    def dims(s, shared):
        return L.Dims(batch=B, num_heads=w.heads, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                      nope_dim=w.nope, v_dim=w.v, s_q=s, dtype=code, rope_shared=shared)

    def ws(d, path):
        n = L.gqla_workspace_bytes(d, path, nbs, max_ctx, NB)
        return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None

    def record(path, s, d, t_med, t_best, kv, flops, bound, extra=None):
        r = {"workload": name, "path": path, "s_q": s, "batch": B, "context": [int(lo), int(hi)],
             "heads": w.heads, "groups": w.groups, "dtype": w.dtype, "ms": t_med * 1e3, "best_ms": t_best * 1e3,
             "tokens_per_s": B * s / t_med, "kv_bytes": kv, "kv_GBps": kv / t_med / 1e9,
             "hbm_frac": kv / t_med / HBM_PEAK, "tflops": flops / t_med / 1e12, "mfma_frac": flops / t_med / MFMA_PEAK,
             "bound": bound, "splits": L.gqla_num_splits(d, L.GQLA_PATH_ABSORB if path == "absorb" else L.GQLA_PATH_GQA,
                                                         nbs, max_ctx, NB)}
        if extra:
            r.update(extra)
        rows.append(r)
        print(json.dumps(r), flush=True)

    # absorb path over the latent cache
    latent = torch.empty(NB, 64, dq, dtype=dt, device="cuda")
    _fill(latent, gen)
    paged = L.Paged(table, lens, max_ctx, NB)
    for s in absorb_sq:
        d = dims(s, 0)
        q_nope = torch.empty(B, s, w.heads, w.nope, dtype=dt, device="cuda")
        q_rope = torch.empty(B, s, w.heads, w.rope, dtype=dt, device="cuda")
        _fill(q_nope, gen)
        _fill(q_rope, gen)
        q_abs = torch.empty(B, s, w.heads, dq, dtype=dt, device="cuda")
        o_lat = torch.empty(B, s, w.heads, w.latent, dtype=torch.float32, device="cuda")
        out = torch.empty(B, s, w.heads, w.v, dtype=dt, device="cuda")
        wsa = ws(d, L.GQLA_PATH_ABSORB)

        def absorb():
            L.gqla_absorb_query(d, q_nope, q_rope, w_uk, q_abs)
            L.gqla_decode_absorb_out(d, paged, q_abs, latent, w_uv, wsa, o_lat, out)

        t_med, t_best = _time(absorb, reps, flush)
        kv = float(ctx.sum()) * dq * elt
        flops = vis(s) * w.heads * 2 * (2 * w.latent + w.rope)
        bound = "mfma" if flops / kv > MFMA_PEAK / HBM_PEAK else "hbm"
        extra = None
        if graph:
            g_med, g_best = _graph_time(absorb, reps, flush)
            extra = {"graph_ms": g_med * 1e3, "graph_best_ms": g_best * 1e3}
        record("absorb", s, d, t_med, t_best, kv, flops, bound, extra)
        del q_nope, q_rope, q_abs, o_lat, out, wsa
    del latent
    torch.cuda.empty_cache()

    # GQA path over a resident expanded cache (filled directly: its values do not change the work)
    shared = rope_shared if (w.rope == 64 and w.dtype == "bf16") else 0
    d0 = dims(gqa_sq[0], shared)
    per_tok = L.gqla_cache_bytes_per_token(d0, L.GQLA_PATH_GQA)
    expanded = torch.empty(NB * 64 * per_tok // elt, dtype=dt, device="cuda")
    _fill(expanded, gen)
    for s in gqa_sq:
        d = dims(s, shared)
        q = torch.empty(B, s, w.heads, w.qk, dtype=dt, device="cuda")
        _fill(q, gen)
        out = torch.empty(B, s, w.heads, w.v, dtype=dt, device="cuda")
        wsg = ws(d, L.GQLA_PATH_GQA)

        def gqa():
            L.gqla_decode_gqa(d, paged, q, expanded, wsg, out)

        t_med, t_best = _time(gqa, reps, flush)
        kv = float(ctx.sum()) * per_tok
        flops = vis(s) * w.heads * 2 * (w.qk + w.v)
        extra = {"gqa_expanded_layout": "shared-rope" if shared else "per-group"}
        if graph:
            g_med, g_best = _graph_time(gqa, reps, flush)
            extra.update({"graph_ms": g_med * 1e3, "graph_best_ms": g_best * 1e3})
        record("gqa", s, d, t_med, t_best, kv, flops, "hbm", extra)
        # append path: the s new tokens of every sequence, latent rows + RoPE + expansion
        # (needs a latent pool too; a small one would not match the block table, so it is
        # timed only where both caches fit next to each other)
        del q, out, wsg
    if NB * 64 * (dq * elt + per_tok) < 120 * 2**30:
        latent = torch.empty(NB, 64, dq, dtype=dt, device="cuda")
        _fill(latent, gen)
        s = gqa_sq[-1]
        d = dims(s, shared)
        c_new = torch.empty(B, s, w.latent, dtype=dt, device="cuda")
        kr_new = torch.empty(B, s, w.rope, dtype=dt, device="cuda")
        _fill(c_new, gen)
        _fill(kr_new, gen)

        def append():
            L.gqla_append_tokens(d, paged, c_new, kr_new, 10000.0, w_uk, w_uv, latent, expanded)

        t_med, t_best = _time(append, reps, flush)
        r = {"workload": name, "path": "append", "s_q": s, "batch": B, "tokens": B * s, "ms": t_med * 1e3,
             "best_ms": t_best * 1e3, "us_per_token": t_med * 1e6 / (B * s),
             "gqa_expanded_layout": "shared-rope" if shared else "per-group"}
        rows.append(r)
        print(json.dumps(r), flush=True)
        del latent
    del expanded
    torch.cuda.empty_cache()
    return rows


def run_output_side(name, reps, gen, flush, s_q=1):
    """The layer's output side after each path at hidden = H * d_v (the module's size):
    absorb: gqla_out_proj (W_UV^g) then W_O, or W_O with W_UV^g folded in, over the fp32
    latent outputs; the GQA path needs only W_O. Weight bytes streamed per call are
    reported as GB/s."""
    from workloads import workload
    w = workload(name)
    if w.dtype != "bf16":
        return []
    B, H = w.batch, w.heads
    hidden = H * w.v
    d = L.Dims(batch=B, num_heads=H, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
               nope_dim=w.nope, v_dim=w.v, s_q=s_q)
    dt = torch.bfloat16
    w_o = torch.empty(hidden, H * w.v, dtype=dt, device="cuda")
    w_uv = torch.empty(w.groups, w.v, w.latent, dtype=dt, device="cuda")
    _fill(w_o, gen, (H * w.v) ** -0.5)
    _fill(w_uv, gen, w.latent ** -0.5)
    w_fold = torch.empty(hidden, H * w.latent, dtype=dt, device="cuda")
    L.gqla_fold_out_weight(d, hidden, w_o, w_uv, w_fold)
    o_lat = torch.empty(B, s_q, H, w.latent, dtype=torch.float32, device="cuda")
    _fill(o_lat, gen)
    out = torch.empty(B, s_q, H, w.v, dtype=dt, device="cuda")
    y = torch.empty(B, s_q, hidden, dtype=dt, device="cuda")
    rows = []
    wo_bytes, wf_bytes = w_o.numel() * 2.0, w_fold.numel() * 2.0
    uv_bytes = w_uv.numel() * 2.0
    cases = (
        ("W_O", lambda: L.gqla_out_hidden(d, hidden, False, out, w_o, y), wo_bytes),
        ("W_UV then W_O", lambda: (L.gqla_out_proj(d, o_lat, w_uv, out), L.gqla_out_hidden(d, hidden, False, out, w_o, y)),
         wo_bytes + uv_bytes),
        ("W_O with W_UV folded", lambda: L.gqla_out_hidden(d, hidden, True, o_lat, w_fold, y), wf_bytes),
    )
    for label, fn, nbytes in cases:
        t_med, t_best = _time(fn, reps, flush)
        r = {"workload": name, "path": "output side", "op": label, "s_q": s_q, "batch": B, "hidden": hidden,
             "ms": t_med * 1e3, "best_ms": t_best * 1e3, "weight_bytes": nbytes, "weight_GBps": nbytes / t_med / 1e9,
             "hbm_frac": nbytes / t_med / HBM_PEAK}
        rows.append(r)
        print(json.dumps(r), flush=True)
    del w_o, w_uv, w_fold, o_lat, out, y
    torch.cuda.empty_cache()
    return rows


def table(rows):
    out = ["| workload | path | s_q | batch | ms (median) | best ms | tokens/s | KV GB/s | % HBM | TFLOP/s | % MFMA | bound | splits |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        if r["path"] in ("append", "output side"):
            continue
        out.append(f"| {r['workload']} | {r['path']} | {r['s_q']} | {r['batch']} | {r['ms']:.3f} | {r['best_ms']:.3f} | "
                   f"{r['tokens_per_s']:,.0f} | {r['kv_GBps']:,.0f} | {r['hbm_frac'] * 100:.1f} | {r['tflops']:.0f} | "
                   f"{r['mfma_frac'] * 100:.1f} | {r['bound']} | {r['splits']} |")
    gr = [r for r in rows if "graph_ms" in r]
    if gr:
        out += ["", "| workload | path | s_q | ms (median) | captured in a HIP graph: ms (median) | best ms | eager minus graph |",
                "|---|---|---|---|---|---|---|"]
        out += [f"| {r['workload']} | {r['path']} | {r['s_q']} | {r['ms']:.4f} | {r['graph_ms']:.4f} | "
                f"{r['graph_best_ms']:.4f} | {(r['ms'] - r['graph_ms']) * 1e3:.1f} us |" for r in gr]
    app = [r for r in rows if r["path"] == "append"]
    if app:
        out += ["", "| workload | append: tokens | ms (median) | us per token |", "|---|---|---|---|"]
        out += [f"| {r['workload']} | {r['tokens']} | {r['ms']:.4f} | {r['us_per_token']:.3f} |" for r in app]
    osd = [r for r in rows if r["path"] == "output side"]
    if osd:
        out += ["", "| workload | output side (s_q = 1) | rows | hidden | ms (median) | weight GB/s | % HBM |",
                "|---|---|---|---|---|---|---|"]
        out += [f"| {r['workload']} | {r['op']} | {r['batch'] * r['s_q']} | {r['hidden']} | {r['ms']:.4f} | "
                f"{r['weight_GBps']:,.0f} | {r['hbm_frac'] * 100:.1f} |" for r in osd]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(CASES))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--output-side", default="llama3-8b-b32-ctx8k,dsv3-b64-ctx8k",
                    help="workloads whose output side (W_O, folded or not) is timed; empty for none")
    ap.add_argument("--out", default=None)
    ap.add_argument("--graph", action="store_true",
                    help="also time each decode path captured in a HIP graph and replayed (graph_ms)")
    ap.add_argument("--block-table", choices=("workload", "identity", "shuffled"), default="workload",
                    help="the workload's block table, or every sequence's blocks adjacent (identity), or a "
                         "seeded permutation of the pool (shuffled)")
    a = ap.parse_args(argv)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2025)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    rows = []
    for name in filter(None, a.workloads.split(",")):
        print(f"[sweep] {name}", file=sys.stderr, flush=True)
        rows += run_workload(name, a.reps, gen, flush, graph=a.graph, block_table=a.block_table)
    for name in filter(None, a.output_side.split(",")):
        print(f"[sweep] output side {name}", file=sys.stderr, flush=True)
        rows += run_output_side(name, a.reps, gen, flush)
    t = table(rows)
    print(t)
    if a.out:
        with open(a.out, "w") as f:
            f.write(t + "\n")
    return rows


if __name__ == "__main__":
    sys.exit(0 if main() else 1)
