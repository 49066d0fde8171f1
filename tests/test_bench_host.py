"""Host logic of bench.py, on the CPU: the rocprofv3 summaries that the
committed profiles and ``roofline.traffic`` come from (kernel traces and
FETCH_SIZE / WRITE_SIZE counter CSVs, here synthetic with known answers),
the traffic figure's tie to the kernel source, and the refusal of more than
one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

HALVES = "void usp::(anonymous namespace)::attn_bf16_kernel<128, 8, 1, 2, 64, true>(usp::(anonymous namespace)::Params)"
MERGE = "void usp::(anonymous namespace)::attn_merge_halves<128, true>(usp::(anonymous namespace)::Params)"
WHOLE_F32 = "void usp::(anonymous namespace)::attn_bf16_kernel<128, 8, 1, 1, 64, false>(usp::(anonymous namespace)::Params)"
LSE = "void usp::(anonymous namespace)::lse_merge_kernel(usp::(anonymous namespace)::MergeParams)"
PACK = "void usp::(anonymous namespace)::relayout_kernel<true>(usp::(anonymous namespace)::RelayoutParams, usp::(anonymous namespace)::Ptrs)"
COPY = "__amd_rocclr_copyBuffer"


def _write_trace(path, dispatches):
    """dispatches: (kernel name, start ns, end ns, workgroups of 256 threads)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
                    "Workgroup_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for name, t0, t1, wgs in dispatches:
            w.writerow([name, t0, t1, wgs * 256, 256, 1, 1])


def test_trace_summary_timed_calls_and_ring_spans(tmp_path):
    # 3 key-half attention calls (the first a warm-up), each with its merge,
    # then a ring pass: two whole-walk blocks that overlap, then the merge
    d = []
    t = 0
    for dur in (5000, 2000, 2200):
        d.append((HALVES, t, t + dur, 1280))
        d.append((MERGE, t + dur + 10, t + dur + 40, 20480))
        t += dur + 100
    d += [(WHOLE_F32, 20000, 22000, 640), (WHOLE_F32, 20100, 22300, 640),
          (LSE, 22400, 22430, 20475)]
    _write_trace(str(tmp_path / "run" / "trace_kernel_trace.csv"), d)
    out = tmp_path / "summary.txt"
    bench.trace_summary([str(tmp_path / "run")], str(out), warmup=1, steps=2)
    text = out.read_text()
    # the timed calls are dispatches 1 and 2: (2.0 + 2.2) / 2 us + 0.03 us of merge
    assert "attn_bf16_kernel 2.1 us + attn_merge_halves 0.0 us = 2.1 us per call" in text
    # first block start (20000) to the merge's end (22430)
    assert "ring passes, kernel time from the first block's start to the merge's end (us), " \
           "in order: 2.4" in text
    assert "attn_bf16_kernel<D=128, whole walks, f32 out> [640 workgroups]: 2.0 2.2" in text
    assert f"attn_bf16.hip sha256 {bench.source_digest()}" in text


def _write_pmc(path, rows):
    """rows: (kernel name, dispatch id, threads, counter, value per instance,
    instances)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for name, disp, threads, ctr, val, inst in rows:
            for _ in range(inst):  # a counter is reported per instance and summed
                w.writerow([disp, name, threads, ctr, val / inst])


def _counter_runs(tmp_path):
    kib = bench.COPY_BYTES / 1024
    fetch = [(COPY, 1, 1 << 26, "FETCH_SIZE", kib / 2, 4), (COPY, 2, 1 << 26, "FETCH_SIZE", kib / 2, 4),
             (COPY, 3, 256, "FETCH_SIZE", 1.0, 1),  # a small copy: not a calibration sample
             (HALVES, 4, 327680, "FETCH_SIZE", 1000.0, 16), (MERGE, 5, 5242880, "FETCH_SIZE", 100.0, 16),
             (PACK, 6, 20971520, "FETCH_SIZE", 327680.0 / 2, 16)]
    write = [(COPY, 11, 1 << 26, "WRITE_SIZE", kib, 4), (HALVES, 14, 327680, "WRITE_SIZE", 500.0, 16),
             (MERGE, 15, 5242880, "WRITE_SIZE", 50.0, 16), (PACK, 16, 20971520, "WRITE_SIZE", 327680.0, 16)]
    _write_pmc(str(tmp_path / "fetch" / "pmc_counter_collection.csv"), fetch)
    _write_pmc(str(tmp_path / "write" / "pmc_counter_collection.csv"), write)
    return [str(tmp_path / "fetch"), str(tmp_path / "write")]


def test_pmc_summary_calibrates_on_the_copy(tmp_path):
    dirs = _counter_runs(tmp_path)
    out = tmp_path / "traffic.json"
    bench.pmc_summary(dirs, str(out))
    res = json.loads(out.read_text())
    # the 1 GiB copy reads half its bytes in FETCH_SIZE KiB, all in WRITE_SIZE KiB
    assert res["fetch_factor"] == pytest.approx(2.0)
    assert res["write_factor"] == pytest.approx(1.0)
    assert res["attention"] == {"read_bytes": pytest.approx(2000 * 1024),
                                "write_bytes": pytest.approx(500 * 1024)}
    assert res["traffic_bytes_per_launch"] == pytest.approx((2000 + 500 + 200 + 50) * 1024)
    assert res["source_sha256"] == bench.source_digest()


def test_relayout_pmc_summary_per_launch_shape(tmp_path):
    dirs = _counter_runs(tmp_path)
    out = tmp_path / "rel.txt"
    bench.relayout_pmc_summary(dirs, str(out))
    line = [ln for ln in out.read_text().splitlines() if ln.startswith("pack[20971520]")][0]
    # 20971520 threads x 16 B = 335.5 MB each way; HBM reads 327680 KiB / 2 x 2
    assert line.split()[1:] == ["1", "335.5", "335.5", "335.5"]


def test_stored_traffic_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"source_sha256": bench.source_digest(),
                                "traffic_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    assert bench.stored_traffic() == 123.0
    path.write_text(json.dumps({"source_sha256": "0" * 64, "traffic_bytes_per_launch": 123.0}))
    assert bench.stored_traffic() is None
    path.write_text("not json")
    assert bench.stored_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
