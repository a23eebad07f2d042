"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the calibration of the
HBM counters against the plain copy, the tie of stored traffic figures to the library
sources, the algorithmic bytes of a decode, and the oracle baseline's report."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

COLUMNS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_csv(path, counter, rows):
    """A counter file in rocprofv3's CSV layout (the columns bench.py reads)."""
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=COLUMNS)
        wr.writeheader()
        for i, (kernel, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                         "Counter_Value": value})


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pmc_collect_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the factors that map the
    same counters onto the known bytes of the calibration copy, then averaged over the
    dispatches of each pass."""
    copy_kib = bench.COPY_ELEMS * 4 / 1024.0
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>"
    fetch = [(mul, copy_kib / 2),                       # the counter reads half the bytes
             ("void sa::fwd_kernel<64>(sa::KArgs)", 1000.0),
             ("void sa::fwd_kernel<64>(sa::KArgs)", 1200.0),
             ("void sa::bwd_kernel<false>(sa::KArgs, void*, int, int)", 3000.0)]
    write = [(mul, copy_kib),
             ("void sa::fwd_kernel<64>(sa::KArgs)", 500.0),
             ("void sa::fwd_kernel<64>(sa::KArgs)", 500.0),
             ("void sa::bwd_kernel<false>(sa::KArgs, void*, int, int)", 700.0)]
    fpath, wpath = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fpath, "FETCH_SIZE", fetch)
    _counter_csv(wpath, "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    bench.pmc_collect("long_8k_s1", str(fpath), str(wpath))
    t = json.loads(out.read_text())
    assert t["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["calibration"]["write_factor"] == pytest.approx(1.0)
    assert t["kernels"]["fwd"]["hbm_bytes"] == pytest.approx(1100.0 * 1024 * 2 + 500.0 * 1024)
    assert t["kernels"]["bwd"]["hbm_bytes"] == pytest.approx(3000.0 * 1024 * 2 + 700.0 * 1024)
    assert t["source_hash"] == bench.source_hash()


def test_traffic_is_reported_only_for_the_current_sources(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(path))
    assert bench.traffic_for("long_8k_s1", "bwd") is None          # no counters taken
    record = {"source_hash": bench.source_hash(), "kernels": {"bwd": {"hbm_bytes": 123.0}}}
    path.write_text(json.dumps(record))
    assert bench.traffic_for("long_8k_s1", "bwd") == 123.0
    assert bench.traffic_for("long_8k_s1", "fwd") is None
    record["source_hash"] = "0" * 64                                 # sources changed since
    path.write_text(json.dumps(record))
    assert bench.traffic_for("long_8k_s1", "bwd") is None


def test_decode_bytes():
    """Each live row: K and V in bf16 per head and its float gate per head; per (b, h) the
    bf16 query and the output."""
    counts = np.array([3, 5])
    H, d = 2, 64
    live = 8
    assert bench.decode_bytes(counts, H, d, 4) == live * H * (2 * d * 2 + 4) + 2 * H * d * (2 + 4)
    assert bench.decode_bytes(counts, H, d, 2) == live * H * (2 * d * 2 + 4) + 2 * H * d * (2 + 2)


def test_cpu_baseline_reports_its_sample():
    """With no time budget the oracle baseline stops after one (entry, head) pair, the entry
    of median length, and says so."""
    w = W.get("tiny_fp32", dtype="bf16")
    data = W.generate(w)
    res = bench.cpu_baseline(data, w, 0.0)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOPS"
    assert res["value"] > 0 and res["cores"] >= 1
    sl = sorted(int(x) for x in data["seqlens"])
    med = sl[len(sl) // 2]
    assert f"1 of {w.H} heads of entry" in res["sample"] and f"(n={med})" in res["sample"]
    assert res["host"]
