"""Decode-attention benchmark of the GQLA hot path on one MI355X.

Default workload: the one-eighth head share of the DeepSeek-V3 layer at real shape (16 query
heads in 2 groups of 8, latent 512 + RoPE 64, d_n = d_v = 128), context 16384, s_q = 2,
batch 10240: the batch whose expanded cache fills 200 GiB with the RoPE key in every group's
K (180 GiB with it once per block). It is the pages' comparison of the GQA path against the
MQA-absorb path at matched resident batch ("GQLA: Group-Query Latent Attention for
Hardware-Adaptive Decoding", Abstract).

The two caches of this batch do not fit in HBM together, so the two paths run one after the
other over the same seeded latent:
  1. GQA path. The latent is drawn on the device chunk by chunk, expanded into the per-group
     K/V cache (gqla_expand_cache) and dropped. One GQA step = gqla_append_tokens of every
     sequence's s_q new tokens into the expanded cache (their K/V in every group; a GQA-only
     deployment keeps no latent cache) + gqla_decode_gqa (+ its split combine).
  2. MQA-absorb path. The expanded cache is freed and the same latent drawn again into the
     latent pool. One absorb step = gqla_append_tokens into the latent cache +
     gqla_absorb_query + gqla_decode_absorb (+ combine) + gqla_out_proj.
Together the two steps are one pass of the whole hot path over the batch.

`value` = the GQA path's decode tokens/s, B * s_q per step, from K back-to-back steps between
two synchronisations; the absorb path at the same batch is under "paths". A second pass of K
steps, each after an untimed 1 GiB read (so that no step finds what it reads in the 256 MiB
last-level cache), gives the median and best step time and, from HIP events recorded around
the decode call on the stream it is launched on, the dominant kernel's launch time for
"roofline" (the GQA split-KV decode). "cpu_baseline" times the fp64 oracle on 16 sampled
sequences of the same batch, read back from the device; per-sequence work is independent, so
its tokens/s is also the rate of the whole batch, whose time is extrapolated and labelled.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--paths gqa,absorb]
       python bench.py --profile        (untimed: a 1 GiB calibration copy, then 3 steps per
                                         path, for rocprofv3 counter passes)
       python bench.py --summarize-pmc FETCH_DIR WRITE_DIR [--store-traffic]
                                        (HBM traffic of the GQA decode from two rocprofv3 --pmc
                                         output folders; --store-traffic records it)
"""
import argparse
import csv
import ctypes
import hashlib
import json
import os
import subprocess
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
CHUNK_BYTES = 1 << 30           # latent drawn and expanded this much at a time


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3-tp8share-ctx16k")
    ap.add_argument("--s-q", type=int, default=None, help="query rows per sequence (default: the workload's largest)")
    ap.add_argument("--absorb-s-q", type=int, default=None, help="absorb path rows (default: --s-q, matched)")
    ap.add_argument("--paths", default="gqa,absorb")
    ap.add_argument("--gqa-layout", choices=("shared-rope", "per-group"), default="shared-rope",
                    help="expanded cache: RoPE key once per block (default) or in every group's K")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-sample", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the fp64 oracle in full on the host-sized workloads (no GPU use) and exit")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--store-traffic", action="store_true")
    return ap.parse_args(argv)


def source_sha(path=DOMINANT_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ HBM traffic records

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
            "dispatches": len(f[gqa[0]]),
            "calibration": {"copy_kernel": big, "bytes": CALIB_BYTES, "fetch_scale": f_scale, "write_scale": w_scale},
            "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -o run -- python3 bench.py "
                         f"--profile --workload {workload_name} --gqa-layout {layout} --paths gqa --no-cpu-baseline",
                         f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -o run -- python3 bench.py "
                         f"--profile --workload {workload_name} --gqa-layout {layout} --paths gqa --no-cpu-baseline",
                         f"python bench.py --summarize-pmc <FETCH_DIR> <WRITE_DIR> --workload {workload_name} "
                         f"--gqa-layout {layout} --store-traffic"]}


def _traffic_entries():
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return []
    return t.get("entries", [t]) if isinstance(t, dict) else []


def store_traffic(entry):
    keep = [e for e in _traffic_entries()
            if (e.get("workload"), e.get("gqa_expanded_layout")) != (entry["workload"], entry["gqa_expanded_layout"])]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"entries": keep + [entry]}, f, indent=1)
        f.write("\n")


def load_traffic(workload_name, layout):
    """Measured traffic of the current GQA decode source on this workload and expanded-cache
    layout, else None."""
    for t in _traffic_entries():
        if (t.get("source_sha256") == source_sha() and t.get("workload") == workload_name
                and t.get("gqa_expanded_layout") == layout):
            return t["traffic_bytes"]
    return None


# ------------------------------------------------------------------ batch and device inputs

def batch_layout(w):
    """Context lengths and block table of the workload's batch, from the same seed streams as
    the host input recipe (lengths: fixed or integer-uniform; table: identity or a seeded
    permutation of the pool)."""
    streams = np.random.SeedSequence(w.seed).spawn(8)
    lo, hi = w.ctx
    B = w.batch
    lens = np.full(B, lo, dtype=np.int64) if lo == hi else np.random.default_rng(streams[6]).integers(lo, hi + 1, size=B)
    nblk = (lens + 63) // 64
    NB = int(nblk.sum())
    phys = (np.random.default_rng(streams[7]).permutation(NB) if w.shuffled else np.arange(NB)).astype(np.int32)
    table = np.full((B, int(nblk.max())), -1, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    for b in range(B):
        table[b, :nblk[b]] = phys[starts[b]:starts[b] + nblk[b]]
    return lens.astype(np.int32), table, NB


class Bench:
    """Seeded device inputs of one batch and the two paths' steps over them."""

    def __init__(self, a, w):
        import torch
        import decode_attention_02_amd as G
        self.torch, self.G, self.a, self.w = torch, G, a, w
        self.s_q = a.s_q or max(w.s_q)
        self.abs_s_q = a.absorb_s_q or self.s_q
        self.lens_h, self.table_h, self.NB = batch_layout(w)
        self.B, self.H = w.batch, w.heads
        self.dq = w.latent + w.rope
        self.blk_bytes = 64 * self.dq * 2
        self.chunk = max(1, CHUNK_BYTES // self.blk_bytes)
        self.table = torch.from_numpy(self.table_h).cuda()
        self.lens = torch.from_numpy(self.lens_h).cuda()
        self.max_ctx = int(self.lens_h.max())
        self.gen = torch.Generator(device="cuda")
        self.seed = w.seed << 8
        mk = dict(batch=self.B, num_heads=self.H, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                  nope_dim=w.nope, v_dim=w.v, dtype=G.GQLA_BF16)
        self.d_gqa = G.Dims(s_q=self.s_q, rope_shared=int(a.gqa_layout == "shared-rope"), **mk)
        self.d_abs = G.Dims(s_q=self.abs_s_q, **mk)
        self.paged = G.Paged(self.table, self.lens, self.max_ctx, self.NB)
        self.w_uk = self.normal((w.groups, w.nope, w.latent), 1, w.latent ** -0.5)
        self.w_uv = self.normal((w.groups, w.v, w.latent), 2, w.latent ** -0.5)
        self.q = self.normal((self.B, self.s_q, self.H, w.qk), 3)                # [q_nope | q_rope]
        self.q_abs_in = self.q if self.abs_s_q == self.s_q else self.normal((self.B, self.abs_s_q, self.H, w.qk), 6)
        self.c_app = self.normal((self.B, max(self.s_q, self.abs_s_q), w.latent), 4)
        self.kr_app = self.normal((self.B, max(self.s_q, self.abs_s_q), w.rope), 5)
        rng = np.random.default_rng(w.seed + 99)
        self.sample = sorted(int(b) for b in rng.choice(self.B, min(a.cpu_sample, self.B), replace=False))
        self.sample_rows = {}   # sequence -> host bf16 bits [blocks][64][d_c + d_R], filled while drawing the latent
        self.sample_done = False

    def normal(self, shape, tag, scale=1.0, out=None):
        torch = self.torch
        self.gen.manual_seed(self.seed + tag)
        t = out if out is not None else torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        return t.normal_(0.0, scale, generator=self.gen)

    def latent_chunks(self, dst=None):
        """Draw the latent pool chunk by chunk (the same values every time): yields (lo, hi,
        chunk tensor [hi - lo][64][d_c + d_R]); with dst the chunks are drawn into it."""
        torch = self.torch
        tmp = None
        for c, lo in enumerate(range(0, self.NB, self.chunk)):
            hi = min(self.NB, lo + self.chunk)
            if dst is not None:
                t = dst[lo:hi]
            else:
                if tmp is None or tmp.shape[0] != hi - lo:
                    tmp = torch.empty((hi - lo, 64, self.dq), dtype=torch.bfloat16, device="cuda")
                t = tmp
            self.normal(None, 16 + c, out=t)
            self.collect_sample(t, lo, hi)
            yield lo, hi, t
        self.sample_done = True

    def collect_sample(self, t, lo, hi):
        if self.a.no_cpu_baseline or self.sample_done:
            return
        for b in self.sample:
            L = int(self.lens_h[b])
            ids = self.table_h[b, :(L + 63) // 64]
            buf = self.sample_rows.setdefault(b, np.zeros(((L + 63) // 64, 64, self.dq), dtype=np.uint16))
            sel = np.nonzero((ids >= lo) & (ids < hi))[0]
            if len(sel):
                idx = self.torch.from_numpy((ids[sel] - lo).astype(np.int64)).cuda()
                buf[sel] = t[idx].view(self.torch.int16).cpu().numpy().view(np.uint16)

    def ws(self, d, path):
        G, torch = self.G, self.torch
        n = G.gqla_workspace_bytes(d, path, self.table.shape[1], self.max_ctx, self.NB)
        return torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda") if n else None

    # --------------------------------------------------------------- GQA path
    def setup_gqa(self):
        torch, G = self.torch, self.G
        per_tok = G.gqla_cache_bytes_per_token(self.d_gqa, G.GQLA_PATH_GQA)
        self.kv_gqa = float(self.lens_h.astype(np.int64).sum()) * per_tok
        log(f"[bench] GQA path: expanded cache {self.NB * 64 * per_tok / 2**30:.1f} GiB ({self.a.gqa_layout})")
        self.expanded = torch.empty(self.NB * 64 * per_tok // 2, dtype=torch.bfloat16, device="cuda")
        dims = self.d_gqa.c()
        lib = G.LIB
        stream = torch.cuda.current_stream().cuda_stream
        t0 = time.time()
        for lo, hi, t in self.latent_chunks():
            ids = torch.arange(lo, hi, dtype=torch.int32, device="cuda")
            # the pool pointer is shifted so that block id `lo` is the chunk's first block;
            # only ids in [lo, hi) are read
            st = lib.gqla_expand_cache(ctypes.byref(dims), ctypes.c_void_p(t.data_ptr() - lo * self.blk_bytes),
                                       ctypes.c_void_p(self.w_uk.data_ptr()), ctypes.c_void_p(self.w_uv.data_ptr()),
                                       ctypes.c_void_p(ids.data_ptr()), hi - lo, self.NB,
                                       ctypes.c_void_p(self.expanded.data_ptr()), ctypes.c_void_p(stream))
            if st != 0:
                raise RuntimeError(f"gqla_expand_cache: {lib.gqla_last_error().decode()}")
        torch.cuda.synchronize()
        log(f"[bench] expanded {self.NB} blocks in {time.time() - t0:.1f} s")
        self.out_g = torch.empty(self.B, self.s_q, self.H, self.w.v, dtype=torch.bfloat16, device="cuda")
        self.lse_g = torch.empty(self.B, self.s_q, self.H, dtype=torch.float32, device="cuda")
        self.ws_g = self.ws(self.d_gqa, G.GQLA_PATH_GQA)
        self.c_app_g = self.c_app[:, :self.s_q].contiguous()
        self.kr_app_g = self.kr_app[:, :self.s_q].contiguous()

    def gqa_step(self, ev=None):
        G = self.G
        if ev: ev[0].record()
        G.gqla_append_tokens(self.d_gqa, self.paged, self.c_app_g, self.kr_app_g, 10000.0, self.w_uk, self.w_uv,
                             None, self.expanded)
        if ev: ev[1].record()
        G.gqla_decode_gqa(self.d_gqa, self.paged, self.q, self.expanded, self.ws_g, self.out_g, self.lse_g)
        if ev: ev[2].record()

    def free_gqa(self):
        del self.expanded, self.out_g, self.lse_g, self.ws_g
        self.torch.cuda.empty_cache()

    # --------------------------------------------------------------- absorb path
    def setup_absorb(self):
        torch, G, w = self.torch, self.G, self.w
        self.kv_abs = float(self.lens_h.astype(np.int64).sum()) * self.dq * 2
        log(f"[bench] absorb path: latent cache {self.NB * self.blk_bytes / 2**30:.1f} GiB")
        self.latent = torch.empty((self.NB, 64, self.dq), dtype=torch.bfloat16, device="cuda")
        for _ in self.latent_chunks(self.latent):
            pass
        s = self.abs_s_q
        self.q_nope = self.q_abs_in[..., :w.nope].contiguous()
        self.q_rope = self.q_abs_in[..., w.nope:].contiguous()
        self.q_abs = torch.empty(self.B, s, self.H, self.dq, dtype=torch.bfloat16, device="cuda")
        self.o_lat = torch.empty(self.B, s, self.H, w.latent, dtype=torch.float32, device="cuda")
        self.out_a = torch.empty(self.B, s, self.H, w.v, dtype=torch.bfloat16, device="cuda")
        self.ws_a = self.ws(self.d_abs, G.GQLA_PATH_ABSORB)
        self.c_app_a = self.c_app[:, :s].contiguous()
        self.kr_app_a = self.kr_app[:, :s].contiguous()
        torch.cuda.synchronize()

    def absorb_step(self, ev=None):
        G = self.G
        if ev: ev[0].record()
        G.gqla_append_tokens(self.d_abs, self.paged, self.c_app_a, self.kr_app_a, 10000.0, self.w_uk, self.w_uv,
                             self.latent, None)
        G.gqla_absorb_query(self.d_abs, self.q_nope, self.q_rope, self.w_uk, self.q_abs)
        if ev: ev[1].record()
        G.gqla_decode_absorb_out(self.d_abs, self.paged, self.q_abs, self.latent, self.w_uv, self.ws_a, self.o_lat,
                                 self.out_a)
        if ev: ev[2].record()

    def free_absorb(self):
        del self.latent, self.q_abs, self.o_lat, self.out_a, self.ws_a
        self.torch.cuda.empty_cache()


def time_path(bn, step, steps, warmup, flush):
    """Pass A: `steps` back-to-back steps between two synchronisations (the step time).
    Pass B: `steps` steps, each after an untimed read of the flush buffer, each with events at
    its start, around its decode call and at its end (median / best step, decode launch)."""
    torch = bn.torch
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s0, s1 = E(), E()
    t0 = time.perf_counter()
    s0.record()
    for _ in range(steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms_a = s0.elapsed_time(s1) / steps
    sink = torch.zeros((), device="cuda")
    marks = []
    for _ in range(steps):
        sink += flush.sum()
        ev = [E() for _ in range(4)]
        step(ev)
        ev[3].record()
        marks.append(ev)
    torch.cuda.synchronize()
    step_ms = sorted(m[0].elapsed_time(m[3]) for m in marks)
    dec_ms = [m[1].elapsed_time(m[2]) for m in marks]
    return {"ms": ms_a, "wall_ms": wall, "median_ms": float(np.median(step_ms)), "best_ms": step_ms[0],
            "decode_ms": float(np.mean(dec_ms)), "decode_best_ms": float(min(dec_ms)),
            "decode_median_ms": float(np.median(dec_ms)),
            "pre_decode_ms": float(np.mean([m[0].elapsed_time(m[1]) for m in marks])),
            "post_decode_ms": float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))}


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2**30, 1)}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        info["clocks"] = {k.strip(" :"): v for k, v in card.items() if "clock" in k.lower()}
    except Exception as e:   # clocks are context only
        info["clocks"] = f"unavailable ({type(e).__name__})"
    return info


def stream_ceilings(torch, gib=4, reps=5):
    """Practical HBM read rates on this GPU, context for the roofline (the published 8 TB/s
    is not reachable by ordinary loads): gqla_stream_read, the library's plain streaming read
    with the decodes' load form, best over a few workgroup counts (the decode's ceiling), and
    two plain torch kernels, a read-only reduction and a copy."""
    import decode_attention_02_amd as G
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def rate(fn, nbytes):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = E(), E()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return nbytes / float(np.median(ts)) / 1e9
    partial = torch.empty(65536, dtype=torch.float32, device="cuda")
    by_wgs = {w: rate(lambda: G.gqla_stream_read(src, partial, w), 4.0 * n) for w in (512, 1024, 2048, 4096, 8192)}
    got = float(partial[:8192].double().sum())
    if got != float(n):   # every fp32 one of the buffer is counted exactly once
        raise RuntimeError(f"gqla_stream_read summed {got} ones, expected {n}")
    best = max(by_wgs, key=by_wgs.get)
    out = {"stream_read_GBps": by_wgs[best], "stream_read_wgs": best,
           "stream_read_by_wgs": {str(k): round(v, 1) for k, v in by_wgs.items()},
           "read_sum_GBps": rate(lambda: src.sum(), 4.0 * n), "copy_GBps": rate(lambda: dst.copy_(src), 8.0 * n),
           "buffer_GiB": gib}
    del src, dst, partial
    torch.cuda.empty_cache()
    return out


def cpu_baseline(bn, budget_s):
    """Time the fp64 oracle (as it stands) on the sampled sequences of the batch, both paths
    per sequence, in passes over the sample until the budget is spent; then one sequence on
    one BLAS thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import gqla_ref as R
    from workloads import bf16_bits_to_f64
    w = bn.w
    torch = bn.torch
    sc = R.qk_scale(w.nope, w.rope)
    host = lambda t: bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))  # noqa: E731
    wk, wv = host(bn.w_uk), host(bn.w_uv)
    seqs = {}
    for b in bn.sample:
        L = int(bn.lens_h[b])
        rows = bf16_bits_to_f64(bn.sample_rows[b].reshape(-1, bn.dq)[:L])
        qg = host(bn.q[b])
        qa = host(bn.q_abs_in[b])
        seqs[b] = (rows[:, :w.latent], rows[:, w.latent:], qg, qa[..., :w.nope], qa[..., w.nope:])

    def gqa(b):
        c, kr, qg, _, _ = seqs[b]
        K, V = R.expand_latent(c, kr, wk, wv)
        R.gqa_attention(qg, K, V, bn.s_q, sc)

    def absorb(b):
        c, kr, _, qn, qr = seqs[b]
        qa = R.absorb_query(qn, qr, wk)
        o_lat, _ = R.absorb_attention(qa, c, kr, bn.abs_s_q, sc)
        R.out_projection(o_lat, wv)

    t_g = t_a = 0.0
    n_g = n_a = 0
    i = 0
    while i < len(bn.sample) or t_g + t_a < budget_s:
        b = bn.sample[i % len(bn.sample)]
        t0 = time.perf_counter()
        gqa(b)
        t1 = time.perf_counter()
        absorb(b)
        t2 = time.perf_counter()
        t_g, t_a, n_g, n_a = t_g + t1 - t0, t_a + t2 - t1, n_g + 1, n_a + 1
        i += 1
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    with threadpool_limits(limits=1):
        b = bn.sample[0]
        t0 = time.perf_counter()
        gqa(b)
        t1 = time.perf_counter()
    gqa_rate = n_g * bn.s_q / t_g
    full_s = t_g / n_g * bn.B
    return {"value": gqa_rate, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"GQA path (expansion of the sequence's latent + grouped attention, s_q={bn.s_q}) on {n_g} "
                      f"decodes of {len(bn.sample)} seeded sample sequences of the batch (context "
                      f"{int(bn.lens_h[bn.sample].min())}-{int(bn.lens_h[bn.sample].max())}), fp64 NumPy, "
                      f"{t_g:.1f} s (the absorb path timed alongside); extrapolated to the whole batch of {bn.B}: {full_s:.0f} s per step",
            "extrapolated_full_batch_s": full_s,
            "absorb_path": {"tokens_per_s": n_a * bn.abs_s_q / t_a, "decodes": n_a, "seconds": t_a,
                            "s_q": bn.abs_s_q},
            "single_thread_gqa_tokens_per_s": bn.s_q / (t1 - t0), "host_cpus": os.cpu_count()}


def cpu_table(names=None, single_thread_upto=1):
    """The fp64 oracle, as it stands, timed in full on the four workloads that fit a host run
    (the tiny layer, LLaMA-3-8B batch 32, DeepSeek-V3 batch 64, the long-context batch 8):
    every sequence of the batch on each path and s_q the workload runs, with all BLAS threads
    and, for the first single_thread_upto + 1 workloads, on one thread too. Inputs are the
    seeded host inputs of each workload (workloads.generate); no GPU is used."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import gqla_ref as R
    from workloads import bf16_bits_to_f64, generate, workload

    def f64(a):
        return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    runs = {"tiny-fp32": [("absorb", 1), ("gqa", 1), ("naive", 1), ("absorb", 2), ("gqa", 2), ("naive", 2)],
            "llama3-8b-b32-ctx8k": [("absorb", 1), ("gqa", 2)],
            "dsv3-b64-ctx8k": [("absorb", 1), ("gqa", 1), ("absorb", 2), ("gqa", 2)],
            "dsv3-b8-ctx32k-64k": [("absorb", 2), ("gqa", 2)]}
    if names is not None:
        runs = {n: runs[n] for n in names}
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    rows = []
    for wi, (name, cases) in enumerate(runs.items()):
        w = workload(name)
        sc = R.qk_scale(w.nope, w.rope)
        for s_q in sorted({c[1] for c in cases}):
            x = generate(w, s_q)
            wk, wv = f64(x.w_uk), f64(x.w_uv)
            seqs = [(f64(x.c_kv_seq[b]), f64(x.k_rope_seq[b]), f64(x.q_nope[b]), f64(x.q_rope[b]))
                    for b in range(len(x.ctx_lens))]

            def one(path, c, kr, qn, qr):
                if path == "gqa":
                    K, V = R.expand_latent(c, kr, wk, wv)
                    R.gqa_attention(np.concatenate([qn, qr], axis=-1), K, V, s_q, sc)
                elif path == "absorb":
                    o_lat, _ = R.absorb_attention(R.absorb_query(qn, qr, wk), c, kr, s_q, sc)
                    R.out_projection(o_lat, wv)
                else:
                    R.mla_expanded_attention(c, kr, wk, wv, qn, qr, s_q, sc)

            for path, sq in cases:
                if sq != s_q:
                    continue
                for nthr in ([threads, 1] if wi <= single_thread_upto else [threads]):
                    with threadpool_limits(limits=nthr):
                        t0 = time.perf_counter()
                        for sqn in seqs:
                            one(path, *sqn)
                        t = time.perf_counter() - t0
                    r = {"workload": name, "path": path, "s_q": s_q, "batch": len(seqs),
                         "context": [int(x.ctx_lens.min()), int(x.ctx_lens.max())], "threads": nthr,
                         "seconds": t, "tokens_per_s": len(seqs) * s_q / t}
                    rows.append(r)
                    log(f"[cpu-table] {name} {path} s_q={s_q} threads={nthr}: {t:.2f} s, {r['tokens_per_s']:.1f} tokens/s")
            del x, seqs
    return {"kind": "oracle", "unit": "tokens/s", "cores": int(threads), "host_cpus": os.cpu_count(),
            "note": "fp64 NumPy oracle over every sequence of each batch (not sampled), seeded host inputs",
            "rows": rows}


def path_record(bn, name, r, kv, flops, s_q, splits):
    ms = r["ms"]
    d = {"s_q": s_q, "ms": ms, "median_ms": r["median_ms"], "best_ms": r["best_ms"], "wall_ms": r["wall_ms"],
         "tokens_per_s": bn.B * s_q / (ms / 1e3), "kv_bytes": kv, "kv_GBps": kv / (ms / 1e3) / 1e9,
         "hbm_frac": kv / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "flops": flops,
         "mfma_frac": flops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
         "decode_ms": r["decode_ms"], "decode_kv_GBps": kv / (r["decode_ms"] / 1e3) / 1e9,
         "decode_hbm_frac": kv / (r["decode_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, "splits": splits}
    if name == "gqa":
        d["step"] = "gqla_append_tokens (expanded cache only) + gqla_decode_gqa"
        d["append_ms"] = r["pre_decode_ms"]
    else:
        d["step"] = ("gqla_append_tokens (latent cache) + gqla_absorb_query + gqla_decode_absorb_out (decode, then "
                     "the split combine fused with W_UV^g)")
        d["append_and_query_ms"] = r["pre_decode_ms"]
        d["decode_includes"] = "the split combine and the W_UV^g value projection"
    return d


def main(argv=None):
    a = parse(argv)
    if a.summarize_pmc:
        t = summarize_pmc(*a.summarize_pmc, a.workload, a.gqa_layout)
        if a.store_traffic:
            store_traffic(t)
        print(json.dumps(t, indent=1))
        return
    if a.cpu_table:
        print(json.dumps({"cpu_table": cpu_table()}), flush=True)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (the library has no "
              "multi-GPU path; the GQA path would shard its groups across ranks)", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import workload

    torch.cuda.set_device(0)
    w = workload(a.workload)
    paths = [p for p in a.paths.split(",") if p]
    log(f"[bench] {w.name}: B={w.batch}, ctx={w.ctx}, H={w.heads}, G={w.groups}, paths {paths}")
    bn = Bench(a, w)
    G = bn.G
    flush = torch.ones(a.flush_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    ctx = bn.lens_h.astype(np.int64)
    vis = lambda s_q: float(sum(int(L) * s_q - s_q * (s_q - 1) // 2 for L in ctx))  # noqa: E731
    res_paths, timing = {}, {}
    info = None if a.profile else device_info(torch)
    ceil = None if a.profile else stream_ceilings(torch)

    if a.profile:   # untimed passes for rocprofv3 counters: calibration copy, then steps
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
        torch.cuda.synchronize()
    if "gqa" in paths:
        bn.setup_gqa()
        n_split = G.gqla_num_splits(bn.d_gqa, G.GQLA_PATH_GQA, bn.table.shape[1], bn.max_ctx, bn.NB)
        if a.profile:
            for _ in range(3):
                bn.gqa_step()
            torch.cuda.synchronize()
        else:
            log(f"[bench] GQA path: warmup {a.warmup}, {a.steps} timed steps x2 (splits {n_split})")
            r = time_path(bn, bn.gqa_step, a.steps, a.warmup, flush)
            timing["gqa"] = r
            res_paths["gqa"] = path_record(bn, "gqa", r, bn.kv_gqa, vis(bn.s_q) * w.heads * 2 * (w.qk + w.v),
                                           bn.s_q, n_split)
            log(f"[bench] GQA step {r['ms']:.3f} ms (median {r['median_ms']:.3f}, best {r['best_ms']:.3f}); "
                f"decode {r['decode_ms']:.3f} ms = {bn.kv_gqa / r['decode_ms'] / 1e6:.0f} GB/s")
        bn.free_gqa()
    if "absorb" in paths:
        bn.setup_absorb()
        n_split = G.gqla_num_splits(bn.d_abs, G.GQLA_PATH_ABSORB, bn.table.shape[1], bn.max_ctx, bn.NB)
        if a.profile:
            for _ in range(3):
                bn.absorb_step()
            torch.cuda.synchronize()
        else:
            log(f"[bench] absorb path: warmup {a.warmup}, {a.steps} timed steps x2 (splits {n_split})")
            r = time_path(bn, bn.absorb_step, a.steps, a.warmup, flush)
            timing["absorb"] = r
            res_paths["absorb"] = path_record(bn, "absorb", r, bn.kv_abs,
                                              vis(bn.abs_s_q) * w.heads * 2 * (2 * w.latent + w.rope),
                                              bn.abs_s_q, n_split)
            log(f"[bench] absorb step {r['ms']:.3f} ms (median {r['median_ms']:.3f}, best {r['best_ms']:.3f}); "
                f"decode {r['decode_ms']:.3f} ms = {bn.kv_abs / r['decode_ms'] / 1e6:.0f} GB/s")
        bn.free_absorb()
    if a.profile:
        log("[bench] profile passes done")
        return

    head = "gqa" if "gqa" in res_paths else "absorb"
    hp = res_paths[head]
    res = {
        "metric": "decode attention tokens/s + KV-read HBM GB/s (% of peak), per path, at batch x context",
        "value": hp["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": hp["ms"],
        "median_ms_per_step": hp["median_ms"], "best_ms_per_step": hp["best_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian inputs drawn on the device)",
        "headline_path": head,
        "config": {"workload": w.name, "batch": bn.B, "context": [int(ctx.min()), int(ctx.max())], "heads": w.heads,
                   "groups": w.groups, "latent": w.latent, "rope": w.rope, "nope": w.nope, "v": w.v,
                   "s_q": {"gqa": bn.s_q, "absorb": bn.abs_s_q}, "gqa_expanded_layout": a.gqa_layout,
                   "block_table": "shuffled" if w.shuffled else "identity", "block_size": 64,
                   "pool_blocks": bn.NB},
        "paths": res_paths,
        "flush": f"untimed read of {a.flush_mib} MiB before each step of the median/best pass",
        "device": info, "stream_ceilings": ceil,
    }
    if "gqa" in timing:
        t = timing["gqa"]
        achieved = bn.kv_gqa / (t["decode_ms"] / 1e3) / 1e9
        res["roofline"] = {"kernel": "gqa_decode_split (gqla_decode_gqa)", "bound": "hbm", "achieved": achieved,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "traffic": load_traffic(w.name, a.gqa_layout), "algorithmic_bytes_per_launch": bn.kv_gqa,
                           "avg_launch_ms": t["decode_ms"], "median_launch_ms": t["decode_median_ms"],
                           "best_launch_ms": t["decode_best_ms"], "launches_timed": a.steps,
                           "splits": res_paths["gqa"]["splits"]}
        if ceil:   # the same rate against what a plain streaming read of this GPU reaches
            res["roofline"]["frac_of_stream_read"] = achieved / ceil["stream_read_GBps"]
    if not a.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle for ~{a.cpu_seconds:.0f} s on {len(bn.sample)} sampled sequences")
        res["cpu_baseline"] = cpu_baseline(bn, a.cpu_seconds)
        if head == "absorb":
            res["cpu_baseline"]["value"] = res["cpu_baseline"]["absorb_path"]["tokens_per_s"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
