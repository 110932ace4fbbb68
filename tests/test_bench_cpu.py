"""CPU: the measurement helpers of bench.py (no device).

The algorithmic bytes the bench divides by, the HBM-traffic summary it reads back from
the rocprofv3 counter runs (FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a 1 GiB
calibration copy, restricted to the timed workload's launches), the staleness guard of
that summary, and the refusal of a multi-GPU run.
"""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from decode_attention_split_amd.workloads import LayerGeom  # noqa: E402
from decode_attention_split_amd import api  # noqa: E402


def test_layer_bytes_by_hand():
    # sliding: 2 KV heads, hd 8, window 4: rows keep min(ctx, 4) keys, K and V
    g = LayerGeom(4, 2, 8, api.RING, 4, 4, False, 0.0, 1.0)
    ctx = np.array([1, 3, 9], np.int32)
    b = bench.layer_bytes(g, 3, ctx)
    kv = (1 + 3 + 4) * 2 * 8 * 2 * 2
    assert b["kv"] == kv
    assert b["decode"] == kv + 3 * 4 * 8 * 2 + 3 * 4 * 8 * 4 + 2 * 3 * 4
    assert b["append"] == 2 * 3 * 2 * 8 * 2 * 2 + 3 * 4
    # global K = V: one tensor, every position
    g = LayerGeom(16, 1, 16, api.LINEAR, 64, 0, True, 0.0, 1.0)
    b = bench.layer_bytes(g, 3, ctx)
    assert b["kv"] == (1 + 3 + 9) * 1 * 16 * 2
    assert b["append"] == 2 * 3 * 1 * 16 * 2 + 3 * 4


def _counter_csv(path, counter, rows):
    fields = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
              "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (kernel, grid, kib) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Grid_Size": grid,
                        "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": kib})


def test_counter_summary_keeps_the_timed_launches_and_scales_by_the_copy(tmp_path, capsys):
    kern = "void ga::(anonymous namespace)::decode_mfma_kernel<false, false, false>(ga::DecodeArgs)"
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = (1 << 30) / 1024.0
    # the copy's FETCH_SIZE reads half its bytes (calibration 2), WRITE_SIZE all of them;
    # the step's launches (grid 65536, three) and another workload's (grid 131072, one)
    fetch = [(copy, 1024, gib_kib / 2), (kern, 65536, 1000.0), (kern, 65536, 1100.0),
             (kern, 65536, 1200.0), (kern, 131072, 9999.0)]
    write = [(copy, 1024, gib_kib), (kern, 65536, 10.0), (kern, 65536, 20.0),
             (kern, 65536, 30.0), (kern, 131072, 999.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    bench.summarize_counters(str(f), str(w), "cmd", "decode_mfma_kernel<false, false, false>")
    out = dict(line.split(": ", 1) for line in capsys.readouterr().out.splitlines()
               if ": " in line and not line.startswith("#"))
    assert out["grid_size"].startswith("65536")
    fetch_b = 1100.0 * 1024 * 2.0  # mean of the grid-65536 launches, times the calibration
    write_b = 20.0 * 1024 * 1.0
    assert float(out["fetch_bytes_per_launch"]) == pytest.approx(fetch_b, rel=1e-6)
    assert float(out["write_bytes_per_launch"]) == pytest.approx(write_b, rel=1e-6)
    assert float(out["hbm_bytes_per_launch"]) == pytest.approx(fetch_b + write_b, rel=1e-6)
    assert out["sources"].split() == bench.TRAFFIC_SOURCES["decode_mfma_kernel"]


def test_traffic_figure_is_dropped_when_its_sources_change(tmp_path, monkeypatch):
    files = bench.traffic_sources("decode_valu_kernel<256, 2, 4>")
    good = ("kernel: x\nhbm_bytes_per_launch: 123\n"
            f"sources: {' '.join(files)}\nsources_sha256: {bench.sources_digest(files)}\n")
    (tmp_path / "hbm_traffic_ok.txt").write_text(good)
    (tmp_path / "hbm_traffic_stale.txt").write_text(good.replace(bench.sources_digest(files),
                                                                 "0" * 64))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("ok") == 123.0
    assert bench.read_traffic("stale") is None
    assert bench.read_traffic("absent") is None
    with pytest.raises(KeyError):
        bench.traffic_sources("some_other_kernel")


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
