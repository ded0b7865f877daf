"""Host-side tools on the CPU: bench.py's single-GPU contract and the rocprofv3 traffic summary."""
import csv
import os
import subprocess
import sys

import pytest

from mha_mla_kv_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_calibrates_on_the_large_copies_only(tmp_path):
    """The copy kernel also serves small uploads; only the 1 GiB copies calibrate the counters."""
    gib = 1 << 30
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    small = [("__amd_rocclr_copyBuffer", v) for v in (1.5, 3.0, 16.0, 2.0, 1.0, 7.0, 5.0)]
    _counters(fetch, "FETCH_SIZE", small + [("__amd_rocclr_copyBuffer", gib / 2 / 1024)] * 4
              + [("void k<1>(Args)", 1000.0)] * 3)
    _counters(write, "WRITE_SIZE", small + [("__amd_rocclr_copyBuffer", gib / 1024)] * 4
              + [("void k<1>(Args)", 10.0)] * 3)
    t = profiling.traffic(str(fetch), str(write), "k<1>", gib)
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert t["read_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2)
    assert t["write_bytes_per_launch"] == pytest.approx(10.0 * 1024)
