"""CPU checks of the C ABI: the library loads, exports every function that
include/sgb.h declares, its structs have the header's layout, and host-side
argument checks reject bad plans before any device call."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import sparse_gradient_backward_amd as sgb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_declared_function_is_exported():
    declared = sgb.header_functions()
    assert set(declared) == {"sgb_plan_create", "sgb_plan_destroy", "sgb_workspace_bytes",
                             "sgb_backward", "sgb_backward_timed", "sgb_backward_noalloc",
                             "sgb_prepare", "sgb_apply", "sgb_device_status",
                             "sgb_runs_view_get", "sgb_status_string", "sgb_forward"}
    lib = ctypes.CDLL(sgb.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sgb.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in declared:
        assert f" T {name}" in out, f"{name} not a defined dynamic symbol"


def test_atomic_library_exports_its_header():
    """libsgb_atomic.so (the atomic scatter-add baseline) exports what
    include/sgb_atomic.h declares, and rejects bad arguments on the host."""
    import sparse_gradient_backward_amd.atomic as atomic
    declared = atomic.header_functions()
    assert declared == ["sgb_atomic_backward"]
    out = subprocess.run(["nm", "-D", "--defined-only", atomic.LIB_PATH], capture_output=True,
                         text=True).stdout
    for name in declared:
        assert f" T {name}" in out, f"{name} not a defined dynamic symbol"
    f = atomic._lib.sgb_atomic_backward
    # argument errors return before any device call
    assert f(0, None, None, None, 8, 0, 0, None, 0, None, 0, None, 1, None, None, 1.0, 0,
             None) == 1
    p = ctypes.c_void_p(16)
    assert f(1, p, p, p, 6, 0, 0, p, 0, p, 0, p, 1, None, p, 1.0, 0, None) == 1   # D % 4
    assert f(2, p, p, p, 8, 0, 2, p, 0, p, 0, None, 0, None, p, 1.0, 0, None) == 2  # nobag, T>1
    assert f(1, p, p, p, 8, 0, 0, p, 0, p, 0, None, 1, None, p, 1.0, 0, None) == 1  # no offsets


def test_struct_layout_matches_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "sgb.h"
#define F(s, m) printf(#s "." #m " %zu\n", offsetof(s, m))
int main(void) {
  printf("sgb_batch %zu\n", sizeof(sgb_batch));
  F(sgb_batch, grad_output); F(sgb_batch, grad_dtype); F(sgb_batch, indices);
  F(sgb_batch, num_indices); F(sgb_batch, offsets); F(sgb_batch, B);
  F(sgb_batch, per_sample_weights);
  printf("sgb_update %zu\n", sizeof(sgb_update));
  F(sgb_update, mode); F(sgb_update, weights); F(sgb_update, momentum); F(sgb_update, grad);
  F(sgb_update, accumulate); F(sgb_update, lr); F(sgb_update, eps);
  F(sgb_update, weights_dtype); F(sgb_update, stochastic_rounding); F(sgb_update, sr_seed);
  F(sgb_update, sr_offset);
  printf("sgb_runs_view %zu\n", sizeof(sgb_runs_view));
  F(sgb_runs_view, sorted_packed); F(sgb_runs_view, info_bits); F(sgb_runs_view, unique_ids);
  F(sgb_runs_view, run_lengths); F(sgb_runs_view, cumulative); F(sgb_runs_view, num_runs);
  F(sgb_runs_view, long_run_ids); F(sgb_runs_view, num_long_run_ids);
  printf("sgb_lookups %zu\n", sizeof(sgb_lookups));
  F(sgb_lookups, indices); F(sgb_lookups, num_indices); F(sgb_lookups, offsets);
  F(sgb_lookups, B); F(sgb_lookups, per_sample_weights);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "layout")
        subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        lines = subprocess.check_output([exe], text=True).split("\n")
    c_layout = dict(l.rsplit(" ", 1) for l in lines if l)
    for name, cls in (("sgb_batch", sgb._Batch), ("sgb_update", sgb._Update),
                      ("sgb_runs_view", sgb._RunsView), ("sgb_lookups", sgb._Lookups)):
        assert int(c_layout[name]) == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert int(c_layout[f"{name}.{field}"]) == getattr(cls, field).offset, (name, field)


def test_status_strings():
    for code in range(8):
        assert sgb.sgb_status_string(code).startswith("SGB_")
    assert sgb.sgb_status_string(99) == "SGB_UNKNOWN_STATUS"


@pytest.mark.parametrize("hsc,doff,pool,thr", [
    ([0, 10], [0, 6], "sum", 4),              # D % 4 != 0
    ([0, 10], [0, 0], "sum", 4),              # D = 0
    ([0, 10], [0, 16384], "sum", 4),          # D above the maximum
    ([0, 10, 10], [0, 8, 16], "sum", 4),      # empty table
    ([1, 10], [0, 8], "sum", 4),              # hash_size_cumsum[0] != 0
    ([0, 10], [0, 8], "sum", 0),              # threshold < 1
    ([0, 10, 20], [0, 8, 24], "none", 4),     # nobag tables must share D
])
def test_plan_argument_errors(hsc, doff, pool, thr):
    with pytest.raises(sgb.SgbError) as e:
        sgb.sgb_plan_create(np.array(hsc), np.array(doff), pool, thr)
    assert e.value.name == "SGB_ERR_INVALID_ARGUMENT"


def test_null_arguments():
    lib = ctypes.CDLL(sgb.LIB_PATH)
    lib.sgb_backward.restype = ctypes.c_int
    lib.sgb_workspace_bytes.restype = ctypes.c_int
    assert lib.sgb_backward(None, None, None, None, ctypes.c_size_t(0), None) == \
        sgb.SGB_ERR_INVALID_ARGUMENT
    assert lib.sgb_workspace_bytes(None, ctypes.c_int64(10), 1, None) == \
        sgb.SGB_ERR_INVALID_ARGUMENT
    lib.sgb_prepare.restype = ctypes.c_int
    lib.sgb_apply.restype = ctypes.c_int
    assert lib.sgb_prepare(None, None, None, ctypes.c_size_t(0), None) == \
        sgb.SGB_ERR_INVALID_ARGUMENT
    assert lib.sgb_apply(None, None, None, None, ctypes.c_size_t(0), None) == \
        sgb.SGB_ERR_INVALID_ARGUMENT
    lib.sgb_plan_destroy(None)
