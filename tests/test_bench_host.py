"""Host-side checks of the benchmark that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    # the benchmark runs on one GPU; asking for more exits before touching a device
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == 2


def test_workload_flops_closed_form():
    # 4 * S^2 * d * H for the kernel point; block-diagonal sum over the images of a batch
    assert WORKLOADS["kernel"].flops() == 4.0 * 8192 ** 2 * 128 * 16
    assert WORKLOADS["4k"].flops() == 3 * 4.0 * 32400 ** 2 * 128 * 16
    assert WORKLOADS["dit"].flops() == 4.0 * 57600 ** 2 * 128 * 40
    assert WORKLOADS["kernel"].elements() == 8192 * 16 * 128
