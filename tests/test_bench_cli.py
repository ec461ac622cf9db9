"""CPU checks of bench.py's command line: more than one GPU is refused with a
message, and the short-run stage names the kernels that serve it."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_short_stage_kernel_names():
    import bench
    assert bench.short_kernels(np.array([16, 128])) == "k_reduce_short8"
    assert bench.short_kernels(np.array([4096])) == "k_reduce_wide"
    assert bench.short_kernels(np.array([64, 1024])) == "k_reduce_short8+k_reduce_wide"
