"""Decode-attention benchmark of the GQLA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic, seeded input:
  1. gqla_append_tokens of each sequence's s_q = 2 new tokens: their latent rows with the
     key rotated to its position, and their expansion into every group's K/V (the
     expansion the GQA path needs, for exactly the tokens that are new),
  2. MQA-absorb path at s_q = 1: gqla_absorb_query -> gqla_decode_absorb -> gqla_out_proj,
  3. GQA path at s_q = 2:        gqla_decode_gqa over the expanded cache.
`value` = decode tokens produced per second by the step (B*1 absorb + B*2 GQA tokens),
from K back-to-back steps between one pair of HIP events. A second pass of K steps records
events between the paths: per-path tokens/s and KV-read GB/s are reported under "paths",
and "roofline" covers the dominant kernel (the GQA split-KV decode), timed with those
events on the stream it runs on. "cpu_baseline" times the fp64 oracle on a bounded sample
of the same batch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --profile            (untimed: a 1 GiB calibration copy, then steps,
                                             for rocprofv3 counter passes)
       python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   (HBM traffic of the GQA decode
                                             from two rocprofv3 --pmc output folders)
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
DOMINANT_SRC = os.path.join(ROOT, "decode_attention_02_amd", "csrc", "gqa_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gqa_decode_split_traffic.json")
CALIB_BYTES = 1 << 30           # plain copy used to scale FETCH_SIZE / WRITE_SIZE


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3-8b-b32-ctx8k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--absorb-sq", type=int, default=1)
    ap.add_argument("--gqa-sq", type=int, default=2)
    ap.add_argument("--gqa-layout", choices=("shared-rope", "per-group"), default="shared-rope",
                    help="expanded cache: RoPE key once per block (default) or in every group's K")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    return ap.parse_args()


def source_sha(path=DOMINANT_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def summarize_pmc(fetch_dir, write_dir, workload_name, layout):
    """Per-dispatch HBM traffic of the GQA decode kernel from FETCH_SIZE / WRITE_SIZE
    passes, each scaled by what the counter reads for the 1 GiB calibration copy."""
    def per_kernel(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        disp = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0   # KiB -> bytes
        out = {}
        for (name, _), v in disp.items():
            out.setdefault(name, []).append(v)
        return out
    f, wr = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in f if "copy" in k.lower() or "elementwise" in k.lower()]
    gqa = [k for k in f if "gqa_decode_split" in k]
    if not copy or not gqa:
        raise SystemExit(f"kernels not found: {list(f)}")
    big = max(copy, key=lambda k: max(f[k]))
    f_scale = CALIB_BYTES / max(f[big])                 # copy reads CALIB_BYTES
    w_scale = CALIB_BYTES / max(wr.get(big, [0.0]))     # and writes CALIB_BYTES
    fetch = float(np.mean(f[gqa[0]])) * f_scale
    write = float(np.mean(wr[gqa[0]])) * w_scale
    return {"workload": workload_name, "gqa_expanded_layout": layout, "kernel": gqa[0], "source_sha256": source_sha(),
            "fetch_bytes": fetch, "write_bytes": write, "traffic_bytes": fetch + write,
            "raw_fetch_bytes": float(np.mean(f[gqa[0]])), "raw_write_bytes": float(np.mean(wr[gqa[0]])),
            "calibration": {"copy_kernel": big, "bytes": CALIB_BYTES, "fetch_scale": f_scale, "write_scale": w_scale},
            "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -o run -- python3 bench.py --profile",
                         "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -o run -- python3 bench.py --profile",
                         "python bench.py --summarize-pmc <FETCH_DIR> <WRITE_DIR>"]}


def load_traffic(workload_name, layout):
    """Measured traffic of the current GQA decode source on this workload and expanded-cache
    layout, else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if (t.get("source_sha256") != source_sha() or t.get("workload") != workload_name
            or t.get("gqa_expanded_layout") != layout):
        return None
    return t["traffic_bytes"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(x, q_abs_sq, gqa_sq, budget_s):
    """Time the fp64 oracle (as it stands) on whole sequences of the batch, in passes over
    the batch, until the budget is spent: absorb path at q_abs_sq rows plus GQA path at
    gqa_sq rows."""
    from threadpoolctl import threadpool_info
    from oracle import gqla_ref as R
    from workloads import queries_for
    w = x.w
    sc = R.qk_scale(w.nope, w.rope)
    wk, wv = x.f64(x.w_uk), x.f64(x.w_uv)
    qn1, qr1 = queries_for(x, q_abs_sq)
    qg = x.f64(x.q)
    done, tokens, t_total = 0, 0, 0.0
    n_seq = len(x.ctx_lens)
    while done == 0 or t_total < budget_s:
        b = done % n_seq
        c, kr = x.f64(x.c_kv_seq[b]), x.f64(x.k_rope_seq[b])
        qn, qr = x.f64(qn1[b]), x.f64(qr1[b])
        t0 = time.perf_counter()
        qa = R.absorb_query(qn, qr, wk)
        o_lat, _ = R.absorb_attention(qa, c, kr, q_abs_sq, sc)
        R.out_projection(o_lat, wv)
        K, V = R.expand_latent(c, kr, wk, wv)
        R.gqa_attention(qg[b], K, V, gqa_sq, sc)
        t_total += time.perf_counter() - t0
        done += 1
        tokens += q_abs_sq + gqa_sq
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence decodes ({done / n_seq:.1f} passes over the {n_seq} sequences, context "
                      f"{int(x.ctx_lens[0])}), absorb s_q={q_abs_sq} + GQA s_q={gqa_sq} per sequence, fp64 NumPy, "
                      f"{t_total:.1f} s",
            "host_cpus": os.cpu_count()}


def main():
    a = parse()
    if a.summarize_pmc:
        print(json.dumps(summarize_pmc(*a.summarize_pmc, a.workload, a.gqa_layout), indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (this build has no "
              "multi-GPU path; the GQA path would shard its groups across ranks)", file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_attention_02_amd as G
    from workloads import generate, queries_for, workload

    torch.cuda.set_device(0)
    w = workload(a.workload)
    log(f"[bench] generating {w.name} (B={w.batch}, ctx={w.ctx}) ...")
    t0 = time.time()
    x = generate(w, a.gqa_sq)
    qn1, qr1 = queries_for(x, a.absorb_sq)
    log(f"[bench] generated in {time.time() - t0:.1f} s; uploading")

    def dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()

    B, H = w.batch, w.heads
    cache, w_uk, w_uv = dev(x.latent_cache), dev(x.w_uk), dev(x.w_uv)
    q_nope1, q_rope1 = dev(qn1), dev(qr1)
    q_g = dev(x.q)
    table = torch.from_numpy(x.block_table).cuda()
    lens = torch.from_numpy(x.ctx_lens).cuda()
    max_ctx = int(x.ctx_lens.max())
    paged = G.Paged(table, lens, max_ctx, x.num_blocks)
    mk = dict(batch=B, num_heads=H, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
              nope_dim=w.nope, v_dim=w.v, dtype=G.GQLA_BF16)
    d_abs = G.Dims(s_q=a.absorb_sq, **mk)
    d_gqa = G.Dims(s_q=a.gqa_sq, rope_shared=int(a.gqa_layout == "shared-rope"), **mk)

    def workspace(d, path):
        n = G.gqla_workspace_bytes(d, path, table.shape[1], max_ctx, x.num_blocks)
        return torch.zeros(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None

    ws_abs, ws_gqa = workspace(d_abs, G.GQLA_PATH_ABSORB), workspace(d_gqa, G.GQLA_PATH_GQA)
    splits = {"absorb": G.gqla_num_splits(d_abs, 0, table.shape[1], max_ctx, x.num_blocks),
              "gqa": G.gqla_num_splits(d_gqa, 1, table.shape[1], max_ctx, x.num_blocks)}
    per_block = 64 * G.gqla_cache_bytes_per_token(d_gqa, G.GQLA_PATH_GQA) // 2   # bf16 values per block
    expanded = torch.empty(x.num_blocks * per_block, dtype=torch.bfloat16, device="cuda")
    all_ids = torch.arange(x.num_blocks, dtype=torch.int32, device="cuda")
    G.gqla_expand_cache(d_gqa, cache, w_uk, w_uv, all_ids, x.num_blocks, expanded)
    # the s_q newest tokens of every sequence: seeded N(0, 1) latent rows and (unrotated)
    # RoPE keys, appended at positions L - s_q .. L - 1 every step (the same values each time)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 77)
    c_app = torch.randn(B, a.gqa_sq, w.latent, generator=gen, device="cuda").to(torch.bfloat16)
    kr_app = torch.randn(B, a.gqa_sq, w.rope, generator=gen, device="cuda").to(torch.bfloat16)

    q_abs = torch.empty(B, a.absorb_sq, H, w.latent + w.rope, dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty(B, a.absorb_sq, H, w.latent, dtype=torch.float32, device="cuda")
    out_abs = torch.empty(B, a.absorb_sq, H, w.v, dtype=torch.bfloat16, device="cuda")
    out_gqa = torch.empty(B, a.gqa_sq, H, w.v, dtype=torch.bfloat16, device="cuda")
    lse_gqa = torch.empty(B, a.gqa_sq, H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    marks = []

    def step(record):
        ev = [E() for _ in range(4)] if record else None
        if record: ev[0].record()
        G.gqla_append_tokens(d_gqa, paged, c_app, kr_app, 10000.0, w_uk, w_uv, cache, expanded)
        if record: ev[1].record()
        G.gqla_absorb_query(d_abs, q_nope1, q_rope1, w_uk, q_abs)
        G.gqla_decode_absorb(d_abs, paged, q_abs, cache, ws_abs, o_lat)
        G.gqla_out_proj(d_abs, o_lat, w_uv, out_abs)
        if record: ev[2].record()
        G.gqla_decode_gqa(d_gqa, paged, q_g, expanded, ws_gqa, out_gqa, lse_gqa)
        if record:
            ev[3].record()
            marks.append(ev)

    if a.profile:   # untimed passes for rocprofv3 counters: calibration copy, then steps
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
        for _ in range(3):
            step(False)
        torch.cuda.synchronize()
        log("[bench] profile passes done")
        return
    log(f"[bench] warmup {a.warmup} steps, splits {splits}")
    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    # Two timed passes of the same steps. The step time (`value`) comes from one event pair
    # around K back-to-back steps; the per-path times (and the dominant kernel's launch
    # duration for the roofline) from a second pass with events between the paths, which
    # make the stream drain at every record and so lengthen the step they sit in.
    start, end = E(), E()
    log(f"[bench] timing {a.steps} steps")
    start.record()
    for _ in range(a.steps):
        step(False)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / a.steps
    log(f"[bench] timing {a.steps} steps with per-path events")
    start.record()
    for _ in range(a.steps):
        step(True)
    end.record()
    torch.cuda.synchronize()
    ms_step_marked = start.elapsed_time(end) / a.steps
    t_exp = np.mean([m[0].elapsed_time(m[1]) for m in marks])
    t_abs = np.mean([m[1].elapsed_time(m[2]) for m in marks])
    t_gqa = np.mean([m[2].elapsed_time(m[3]) for m in marks])
    log(f"[bench] ms/step {ms_step:.4f} ({ms_step_marked:.4f} with per-path events): append {t_exp:.4f} "
        f"absorb {t_abs:.4f} gqa {t_gqa:.4f}")

    ctx = x.ctx_lens.astype(np.int64)
    elt = 2
    kv_abs = float(ctx.sum() * (w.latent + w.rope) * elt)
    kv_gqa = float(ctx.sum() * G.gqla_cache_bytes_per_token(d_gqa, G.GQLA_PATH_GQA))
    vis = lambda s_q: float(sum(sum(L - s_q + 1 + i for i in range(s_q)) for L in ctx))  # noqa: E731
    fl_abs = vis(a.absorb_sq) * H * 2 * (2 * w.latent + w.rope)
    fl_gqa = vis(a.gqa_sq) * H * 2 * (w.qk + w.v)
    tok_step = B * (a.absorb_sq + a.gqa_sq)
    res = {
        "metric": "decode attention tokens/s + KV-read HBM GB/s (% of peak), per path, at batch x context",
        "value": tok_step / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step,
        "ms_per_step_with_path_events": ms_step_marked,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "context": int(ctx.max()), "heads": H,
                   "groups": w.groups, "latent": w.latent, "rope": w.rope, "nope": w.nope, "v": w.v,
                   "s_q": {"absorb": a.absorb_sq, "gqa": a.gqa_sq},
                   "gqa_expanded_layout": a.gqa_layout,
                   "block_table": "shuffled" if w.shuffled else "identity", "block_size": 64,
                   "splits": splits},
        "paths": {
            "absorb": {"s_q": a.absorb_sq, "ms": t_abs, "tokens_per_s": B * a.absorb_sq / (t_abs / 1e3),
                       "kv_bytes": kv_abs, "kv_GBps": kv_abs / (t_abs / 1e3) / 1e9,
                       "hbm_frac": kv_abs / (t_abs / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "flops": fl_abs, "mfma_frac": fl_abs / (t_abs / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
            "gqa": {"s_q": a.gqa_sq, "ms": t_gqa, "tokens_per_s": B * a.gqa_sq / (t_gqa / 1e3),
                    "kv_bytes": kv_gqa, "kv_GBps": kv_gqa / (t_gqa / 1e3) / 1e9,
                    "hbm_frac": kv_gqa / (t_gqa / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "flops": fl_gqa, "mfma_frac": fl_gqa / (t_gqa / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
            "append": {"tokens": B * a.gqa_sq, "ms": t_exp,
                       "note": "gqla_append_tokens: new latent rows, RoPE, expansion into the groups"},
        },
        "roofline": {"kernel": "gqa_decode_split (gqla_decode_gqa)", "bound": "hbm",
                     "achieved": kv_gqa / (t_gqa / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kv_gqa / (t_gqa / 1e3) / 1e9 / HBM_PEAK_GBS, "traffic": load_traffic(w.name, a.gqa_layout),
                     "algorithmic_bytes_per_launch": kv_gqa, "avg_launch_ms": t_gqa},
    }
    if not a.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle for ~{a.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(x, a.absorb_sq, a.gqa_sq, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
