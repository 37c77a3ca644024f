"""CPU checks of bench.py's host logic: the one-GPU contract and the HBM-traffic summary
(FETCH_SIZE / WRITE_SIZE scaled by what the counters read for the calibration copy)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GQA = "void gqla::(anonymous namespace)::gqa_decode_split<128, 128, 8, 1, true>(gqla::AttnParams)"
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_dir(path, counter, rows):
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    kib = bench.CALIB_BYTES / 1024
    # FETCH_SIZE reads half of what the copy moves, WRITE_SIZE all of it; each dispatch's
    # value arrives split over several rows (one per hardware instance), which are summed.
    _counter_dir(tmp_path / "fetch", "FETCH_SIZE",
                 [(1, COPY, kib / 4), (1, COPY, kib / 4), (2, GQA, 100.0), (2, GQA, 300.0), (3, GQA, 600.0)])
    _counter_dir(tmp_path / "write", "WRITE_SIZE",
                 [(1, COPY, kib), (2, GQA, 8.0), (3, GQA, 12.0)])
    t = bench.summarize_pmc(str(tmp_path / "fetch"), str(tmp_path / "write"), "w", "shared-rope")
    assert t["kernel"] == GQA
    assert t["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["calibration"]["write_scale"] == pytest.approx(1.0)
    assert t["raw_fetch_bytes"] == pytest.approx(500.0 * 1024)          # mean of 400 and 600 KiB
    assert t["fetch_bytes"] == pytest.approx(1000.0 * 1024)
    assert t["write_bytes"] == pytest.approx(10.0 * 1024)
    assert t["traffic_bytes"] == pytest.approx(1010.0 * 1024)
    assert t["source_sha256"] == bench.source_sha()


def test_stored_traffic_is_used_only_for_the_same_source_workload_and_layout(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic("w", "shared-rope") is None                # no file
    good = {"source_sha256": bench.source_sha(), "workload": "w", "gqa_expanded_layout": "shared-rope",
            "traffic_bytes": 123.0}
    f.write_text(json.dumps(good))
    assert bench.load_traffic("w", "shared-rope") == 123.0
    assert bench.load_traffic("other", "shared-rope") is None
    assert bench.load_traffic("w", "per-group") is None
    f.write_text(json.dumps(dict(good, source_sha256="0" * 64)))        # kernel changed since
    assert bench.load_traffic("w", "shared-rope") is None


def test_cpu_table_times_every_case_of_the_tiny_layer():
    """bench.py --cpu-table's oracle timing on the tiny layer: every path and s_q the layer
    runs, on all BLAS threads and on one."""
    import bench
    t = bench.cpu_table(names=["tiny-fp32"])
    assert t["kind"] == "oracle" and t["cores"] >= 1
    got = {(r["path"], r["s_q"], r["threads"]) for r in t["rows"]}
    want = {(p, s, n) for p in ("absorb", "gqa", "naive") for s in (1, 2) for n in {t["cores"], 1}}
    assert got == want
    assert all(r["batch"] == 2 and r["seconds"] > 0 and r["tokens_per_s"] > 0 for r in t["rows"])
