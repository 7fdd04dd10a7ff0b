"""Host logic of bench.py that needs no GPU: the one-GPU guard, the rocprofv3
summary writer, and the scaling of PMC byte counters by the copy probe."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU only" in out.stderr
    assert out.stdout == ""


def test_summarize_stats_writes_the_table(tmp_path):
    src = tmp_path / "kernel_stats.csv"
    with open(src, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void fp4q::(anonymous namespace)::gemm_tile_kernel<0, 0, true>(fp4q::GemmParams)", 3,
                    7500000, 2500000, 90.5, 2400000, 2600000, 1.0])
        w.writerow(["fp4q::(anonymous namespace)::zero_global_kernel(float*)", 2, 4000, 2000, 0.1, 1500, 2500, 1.0])
    md = tmp_path / "out.md"
    bench.summarize_stats(str(src), str(md), "a title", "rocprofv3 --kernel-trace --stats -- python3 bench.py")
    text = md.read_text()
    assert text.startswith("# a title\n")
    assert "rocprofv3 --kernel-trace --stats -- python3 bench.py" in text
    assert "| `gemm_tile_kernel<0, 0, true>` | 3 | 2500.0 | 2400.0 | 2600.0 | 90.50 |" in text
    assert "| `zero_global_kernel` | 2 | 2.0 | 1.5 | 2.5 | 0.10 |" in text


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, v in rows:
            w.writerow([name, counter, v])


def test_traffic_scaling_by_the_copy_probe(tmp_path):
    # the copy probe moves COPY_PROBE_BYTES each way; its counters read 0.5x
    # (fetch) and 1.0x (write) of that, so the GEMM's readings scale by 2 and 1
    kib = bench.COPY_PROBE_BYTES / 1024.0
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    _pmc_csv(f, "FETCH_SIZE", [("gemm_tile_kernel<0, 0, true>", 1000.0), ("gemm_tile_kernel<0, 0, true>", 3000.0),
                               ("quantize_kernel<0, 16, 1, true, true>", 99999.0)])
    _pmc_csv(w, "WRITE_SIZE", [("gemm_tile_kernel<0, 0, true>", 500.0)])
    _pmc_csv(cf, "FETCH_SIZE", [("neg_kernel", 0.5 * kib)])
    _pmc_csv(cw, "WRITE_SIZE", [("neg_kernel", kib)])
    out = tmp_path / "traffic.json"
    rec = bench.traffic_from_pmc("wl", str(f), str(w), str(cf), str(cw), str(out))
    assert rec["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 / 0.5)
    assert rec["write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])
    assert rec["dispatches"] == {"fetch": 2, "write": 1}
    assert out.exists()
