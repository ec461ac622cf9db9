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


def test_path_byte_model_hand_case():
    """The whole-path byte model on a hand-worked batch: one table of 10 rows
    x 8 columns, bags {1, 1, 3} and {0}, sum pooling, fp32 grads, SGD.
    N = 4 lookups, U = 3 rows, no coefficients:
      indices + sorted stream  4 * (8 + 2 * (8 + 4))   = 128
      gather                   4 lookups * 8 * 4 bytes = 128
      offsets                  (2 + 1) * 8             =  24
      runs                     3 * 24                  =  72
      SGD row update           3 rows * 8 * 4 * 2      = 192   -> 544
    and the compulsory bytes: grad_output 2 * 8 * 4 = 64, indices 32, offsets
    24, rows read and written 192 -> 312."""
    import bench
    import synth
    spec = synth.Spec("hand", 1, (10,), (8,), 2, ("fixed", 1), ("uniform",), "sum", False,
                      "f32", "sgd")
    inp = synth.Inputs(spec, 1, 2, np.array([0, 10]), np.array([0, 8], np.int32),
                       np.array([0, 3, 4]), np.array([1, 1, 3, 0]), None,
                       np.zeros((2, 8), np.float32))
    run_D = np.array([8, 8, 8])
    run_len = np.array([1, 2, 1])   # rows 0, 1, 3
    b, b_path, b_comp = bench.stage_bytes(inp, spec, 3, run_D, run_len, 256, 1, 1024)
    assert b_path == 544
    assert b_comp == 312
    assert b["reduce_short"] + b["reduce_long"] >= 128 + 192   # gather + row update
