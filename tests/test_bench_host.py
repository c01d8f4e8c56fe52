"""Host-side checks of bench.py (CPU only): the one-GPU guard and the traffic record lookup."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_only_for_measured_workloads():
    assert bench.measured_traffic("tiny", "gm", "select_kernel") is None
    assert bench.measured_traffic("llama3b_decode", "pl", "select_kernel") is None
    v = bench.measured_traffic("llama3b_decode", "gm", "select_kernel")
    # a number while the kernel sources match the record, None once they change
    assert v is None or (isinstance(v, int) and v > 0)
