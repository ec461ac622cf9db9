"""Python binding of libsgb.so, the gfx950 pooled embedding-bag backward.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/sgb.h``.  The module-level functions
carry the C entry points' names; ``Plan`` is a small convenience wrapper.
PyTorch supplies device memory and the HIP stream.

Importing this package fails loudly (ImportError) when libsgb.so has not been
built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SGB_LIBRARY selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("SGB_LIBRARY") or os.path.join(_HERE, "libsgb.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "sgb.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m sparse_gradient_backward_amd.build` (hipcc, gfx950)")

# torch ships its own HIP runtime.  Load it first so that libsgb.so binds to
# that same runtime (by soname): device pointers and streams come from torch,
# and two HIP runtimes in one process do not share streams or contexts.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes() -> list:
    with open("/proc/self/maps") as f:
        return sorted(set(re.findall(r"(/\S*libamdhip64\S*)", f.read())))


if len(_hip_runtimes()) > 1:
    raise ImportError("more than one HIP runtime is loaded in this process: "
                      f"{_hip_runtimes()}; import torch before any other HIP library")

# ------------------------------------------------------------------ enums

SGB_OK, SGB_ERR_INVALID_ARGUMENT, SGB_ERR_UNSUPPORTED, SGB_ERR_WORKSPACE_TOO_SMALL, \
    SGB_ERR_INDEX_OUT_OF_RANGE, SGB_ERR_BAD_OFFSETS, SGB_ERR_HIP, SGB_ERR_INTERNAL = range(8)
POOLING = {"sum": 0, "mean": 1, "none": 2}
DTYPE = {"f32": 0, "bf16": 1, "int8": 2, "f16": 3}
MODE = {"dense": 0, "sgd": 1, "rowwise_adagrad": 2}


class _Batch(ctypes.Structure):
    _fields_ = [("grad_output", ctypes.c_void_p), ("grad_dtype", ctypes.c_int32),
                ("indices", ctypes.c_void_p), ("num_indices", ctypes.c_int64),
                ("offsets", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("per_sample_weights", ctypes.c_void_p)]


class _Lookups(ctypes.Structure):
    _fields_ = [("indices", ctypes.c_void_p), ("num_indices", ctypes.c_int64),
                ("offsets", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("per_sample_weights", ctypes.c_void_p)]


class _Update(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("weights", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("accumulate", ctypes.c_int32), ("lr", ctypes.c_float), ("eps", ctypes.c_float),
                ("weights_dtype", ctypes.c_int32), ("stochastic_rounding", ctypes.c_int32),
                ("sr_seed", ctypes.c_uint64), ("sr_offset", ctypes.c_uint64)]


class _RunsView(ctypes.Structure):
    _fields_ = [("sorted_packed", ctypes.c_void_p), ("info_bits", ctypes.c_int32),
                ("unique_ids", ctypes.c_void_p), ("run_lengths", ctypes.c_void_p),
                ("cumulative", ctypes.c_void_p), ("num_runs", ctypes.c_void_p),
                ("long_run_ids", ctypes.c_void_p), ("num_long_run_ids", ctypes.c_void_p)]


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_lib.sgb_plan_create.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _vp, _i32, _i32]
_lib.sgb_plan_destroy.argtypes = [_vp]
_lib.sgb_plan_destroy.restype = None
_lib.sgb_workspace_bytes.argtypes = [_vp, _i64, _i32, ctypes.POINTER(ctypes.c_size_t)]
_lib.sgb_backward.argtypes = [_vp, ctypes.POINTER(_Batch), ctypes.POINTER(_Update), _vp,
                              ctypes.c_size_t, _vp]
_lib.sgb_backward_timed.argtypes = [_vp, ctypes.POINTER(_Batch), ctypes.POINTER(_Update), _vp,
                                    ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]
_lib.sgb_backward_noalloc.argtypes = [_vp, ctypes.POINTER(_Batch), ctypes.POINTER(_Update), _vp]
_lib.sgb_prepare.argtypes = [_vp, ctypes.POINTER(_Batch), _vp, ctypes.c_size_t, _vp]
_lib.sgb_apply.argtypes = [_vp, ctypes.POINTER(_Batch), ctypes.POINTER(_Update), _vp,
                           ctypes.c_size_t, _vp]
_lib.sgb_device_status.argtypes = [_vp, _vp, _vp, ctypes.POINTER(_i32)]
_lib.sgb_forward.argtypes = [_vp, ctypes.POINTER(_Lookups), _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.sgb_runs_view_get.argtypes = [_vp, _vp, _i64, _i32, ctypes.POINTER(_RunsView)]
_lib.sgb_status_string.argtypes = [_i32]
_lib.sgb_status_string.restype = ctypes.c_char_p
for _f in ("sgb_plan_create", "sgb_workspace_bytes", "sgb_backward", "sgb_backward_timed",
           "sgb_backward_noalloc", "sgb_prepare", "sgb_apply", "sgb_device_status",
           "sgb_runs_view_get", "sgb_forward"):
    getattr(_lib, _f).restype = ctypes.c_int


class SgbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = sgb_status_string(status)
        super().__init__(f"{where}: {self.name}")


def _check(st: int, where: str):
    if st != SGB_OK:
        raise SgbError(st, where)


def header_functions() -> list:
    """Names of the functions include/sgb.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(sgb_\w+)\s*\(", text, re.M)))


def exported_functions() -> list:
    return [n for n in header_functions() if hasattr(_lib, n)]


# ------------------------------------------------------------------ entry points

def sgb_status_string(status: int) -> str:
    return _lib.sgb_status_string(int(status)).decode()


def sgb_plan_create(hash_size_cumsum, D_offsets, pooling: str = "sum",
                    max_segment_length_per_warp: int = 256) -> int:
    """Returns the plan handle (int).  Host arrays are copied by the library."""
    hsc = np.ascontiguousarray(hash_size_cumsum, dtype=np.int64)
    doff = np.ascontiguousarray(D_offsets, dtype=np.int32)
    T = int(hsc.shape[0]) - 1
    if doff.shape[0] != T + 1:
        raise SgbError(SGB_ERR_INVALID_ARGUMENT, "sgb_plan_create: D_offsets length")
    h = _vp()
    _check(_lib.sgb_plan_create(ctypes.byref(h), T, hsc.ctypes.data, doff.ctypes.data,
                                POOLING[pooling], int(max_segment_length_per_warp)),
           "sgb_plan_create")
    return h.value


def sgb_plan_destroy(plan: int) -> None:
    _lib.sgb_plan_destroy(plan)


def sgb_workspace_bytes(plan: int, num_indices: int, B: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.sgb_workspace_bytes(plan, int(num_indices), int(B), ctypes.byref(n)),
           "sgb_workspace_bytes")
    return int(n.value)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


STAGES = ("linearize", "sort_pass", "sort", "rle", "runs", "fill", "reduce_long",
          "reduce_short")


def sgb_backward(plan: int, grad_output, indices, offsets, B: int, per_sample_weights,
                 mode: str, weights=None, momentum=None, grad=None, accumulate: bool = False,
                 lr: float = 0.0, eps: float = 0.0, workspace=None, stream=None,
                 events=None, stochastic_rounding: bool = False, sr_seed: int = 0,
                 sr_offset: int = 0) -> None:
    """Enqueue one backward pass.  Tensors are device tensors; grad_output is
    float32 or bfloat16, indices/offsets int64, per_sample_weights float32;
    weights float32, or bfloat16 / float16 (SGD / row-wise Adagrad) rounded
    to nearest even or, with stochastic_rounding, stochastically from
    (sr_seed, sr_offset), or uint8 INT8 rows (SGD / row-wise Adagrad: each row its D
    codes then fp32 scale and bias, tables back to back).
    `events`, if given, is a list of 2 * len(STAGES) recorded-once
    torch.cuda.Event(enable_timing=True) objects (or None entries) that the
    library records around each stage (sgb_backward_timed)."""
    batch, upd = _marshal(grad_output, indices, offsets, B, per_sample_weights, mode, weights,
                          momentum, grad, accumulate, lr, eps, stochastic_rounding, sr_seed,
                          sr_offset, "sgb_backward")
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    if events is None:
        _check(_lib.sgb_backward(plan, ctypes.byref(batch), ctypes.byref(upd), ws_ptr, ws_bytes,
                                 _stream(stream)), "sgb_backward")
    else:
        arr = (_vp * (2 * len(STAGES)))(*[None if e is None else int(e.cuda_event)
                                          for e in events])
        _check(_lib.sgb_backward_timed(plan, ctypes.byref(batch), ctypes.byref(upd), ws_ptr,
                                       ws_bytes, _stream(stream), arr), "sgb_backward_timed")


def sgb_backward_noalloc(plan: int, grad_output, indices, offsets, B: int, per_sample_weights,
                         mode: str, weights=None, momentum=None, grad=None,
                         accumulate: bool = False, lr: float = 0.0, eps: float = 0.0,
                         stream=None, stochastic_rounding: bool = False, sr_seed: int = 0,
                         sr_offset: int = 0) -> None:
    """sgb_backward without a workspace: the library's fixed per-GPU scratch
    (64 MiB) serves as one, and nothing is allocated.  Calls that overlap on
    one GPU race; device_status / runs_view read this scratch when given
    workspace=None."""
    batch, upd = _marshal(grad_output, indices, offsets, B, per_sample_weights, mode, weights,
                          momentum, grad, accumulate, lr, eps, stochastic_rounding, sr_seed,
                          sr_offset, "sgb_backward_noalloc")
    _check(_lib.sgb_backward_noalloc(plan, ctypes.byref(batch), ctypes.byref(upd),
                                     _stream(stream)), "sgb_backward_noalloc")


def sgb_prepare(plan: int, indices, offsets, B: int, per_sample_weights, workspace,
                stream=None, grad_output=None) -> None:
    """Enqueue the part of the backward that reads only the lookups
    (linearisation, sort, run-length encoding, long-run list) into
    `workspace`; sgb_apply with the same lookups and workspace finishes it."""
    import torch
    go = grad_output if grad_output is not None else torch.empty(0, dtype=torch.float32)
    batch, _ = _marshal(go, indices, offsets, B, per_sample_weights, "dense", None, None, None,
                        False, 0.0, 0.0, False, 0, 0, "sgb_prepare")
    if grad_output is None:
        batch.grad_output = None
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check(_lib.sgb_prepare(plan, ctypes.byref(batch), _ptr(workspace), ws_bytes,
                            _stream(stream)), "sgb_prepare")


def sgb_apply(plan: int, grad_output, indices, offsets, B: int, per_sample_weights, mode: str,
              weights=None, momentum=None, grad=None, accumulate: bool = False, lr: float = 0.0,
              eps: float = 0.0, workspace=None, stream=None, stochastic_rounding: bool = False,
              sr_seed: int = 0, sr_offset: int = 0) -> None:
    """Enqueue the reductions and row updates of a batch whose lookups
    sgb_prepare has already processed into `workspace` (same arguments as
    sgb_backward)."""
    batch, upd = _marshal(grad_output, indices, offsets, B, per_sample_weights, mode, weights,
                          momentum, grad, accumulate, lr, eps, stochastic_rounding, sr_seed,
                          sr_offset, "sgb_apply")
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check(_lib.sgb_apply(plan, ctypes.byref(batch), ctypes.byref(upd), _ptr(workspace),
                          ws_bytes, _stream(stream)), "sgb_apply")


def _marshal(grad_output, indices, offsets, B, per_sample_weights, mode, weights, momentum, grad,
             accumulate, lr, eps, stochastic_rounding, sr_seed, sr_offset, where):
    import torch
    gd = {torch.float32: "f32", torch.bfloat16: "bf16"}[grad_output.dtype]
    for name, t, dt in (("indices", indices, torch.int64), ("offsets", offsets, torch.int64),
                        ("per_sample_weights", per_sample_weights, torch.float32),
                        ("weights", weights, weights.dtype if weights is not None and
                         weights.dtype in (torch.bfloat16, torch.float16, torch.uint8)
                         else torch.float32),
                        ("momentum", momentum, torch.float32),
                        ("grad", grad, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise SgbError(SGB_ERR_INVALID_ARGUMENT, f"{where}: {name} must be contiguous {dt}")
    if not grad_output.is_contiguous():
        raise SgbError(SGB_ERR_INVALID_ARGUMENT, f"{where}: grad_output must be contiguous")
    batch = _Batch(_ptr(grad_output), DTYPE[gd], _ptr(indices), int(indices.numel()),
                   _ptr(offsets), int(B), _ptr(per_sample_weights))
    wdt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.uint8: "int8"}.get(
        weights.dtype if weights is not None else None, "f32")
    upd = _Update(MODE[mode], _ptr(weights), _ptr(momentum), _ptr(grad), 1 if accumulate else 0,
                  float(lr), float(eps), DTYPE[wdt],
                  1 if stochastic_rounding else 0, int(sr_seed) & (2**64 - 1),
                  int(sr_offset) & (2**64 - 1))
    return batch, upd


def sgb_forward(plan: int, indices, offsets, B: int, per_sample_weights, weights, output,
                workspace, stream=None) -> None:
    """Enqueue the pooled forward (sgb_forward): output [B][sum D] (bag) or
    [N][D] (nobag) float32, from the flat float32 weights.  Device tensors;
    indices/offsets int64, per_sample_weights float32 or None."""
    import torch
    for name, t, dt in (("indices", indices, torch.int64), ("offsets", offsets, torch.int64),
                        ("per_sample_weights", per_sample_weights, torch.float32),
                        ("weights", weights, torch.float32), ("output", output, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise SgbError(SGB_ERR_INVALID_ARGUMENT, f"sgb_forward: {name} must be contiguous {dt}")
    lk = _Lookups(_ptr(indices), int(indices.numel()), _ptr(offsets), int(B),
                  _ptr(per_sample_weights))
    ws_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    _check(_lib.sgb_forward(plan, ctypes.byref(lk), _ptr(weights), _ptr(output), _ptr(workspace),
                            ws_bytes, _stream(stream)), "sgb_forward")


def sgb_device_status(plan: int, workspace, stream=None) -> int:
    out = _i32()
    _check(_lib.sgb_device_status(plan, _ptr(workspace), _stream(stream), ctypes.byref(out)),
           "sgb_device_status")
    return int(out.value)


def sgb_runs_view_get(plan: int, workspace, num_indices: int, B: int) -> dict:
    """Device views (torch tensors into `workspace`) of the run structure."""
    import torch
    v = _RunsView()
    _check(_lib.sgb_runs_view_get(plan, _ptr(workspace), int(num_indices), int(B), ctypes.byref(v)),
           "sgb_runs_view_get")
    base = int(workspace.data_ptr())
    ws = workspace.view(torch.uint8)

    def view(ptr, n, dtype):
        off = int(ptr) - base
        size = torch.empty((), dtype=dtype).element_size()
        return ws[off:off + n * size].view(dtype)

    num_runs = int(view(v.num_runs, 1, torch.int32).item())
    num_long = int(view(v.num_long_run_ids, 1, torch.int64).item())
    return dict(sorted_packed=view(v.sorted_packed, num_indices, torch.int64),
                info_bits=int(v.info_bits), num_runs=num_runs, num_long=num_long,
                unique_ids=view(v.unique_ids, num_runs, torch.int64),
                run_lengths=view(v.run_lengths, num_runs, torch.int32),
                cumulative=view(v.cumulative, num_runs + 1, torch.int32),
                long_run_ids=view(v.long_run_ids, num_long, torch.int32))


class Plan:
    """Owns a plan handle; thin convenience over the entry points above."""

    def __init__(self, hash_size_cumsum, D_offsets, pooling: str = "sum",
                 max_segment_length_per_warp: int = 256):
        self.handle = sgb_plan_create(hash_size_cumsum, D_offsets, pooling,
                                      max_segment_length_per_warp)
        self.pooling = pooling
        self.thr = int(max_segment_length_per_warp)

    def workspace_bytes(self, num_indices: int, B: int) -> int:
        return sgb_workspace_bytes(self.handle, num_indices, B)

    def workspace(self, num_indices: int, B: int, device="cuda"):
        import torch
        return torch.empty(max(self.workspace_bytes(num_indices, B), 256), dtype=torch.uint8,
                           device=device)

    def backward(self, *args, **kw):
        return sgb_backward(self.handle, *args, **kw)

    def backward_noalloc(self, *args, **kw):
        return sgb_backward_noalloc(self.handle, *args, **kw)

    def prepare(self, *args, **kw):
        return sgb_prepare(self.handle, *args, **kw)

    def apply(self, *args, **kw):
        return sgb_apply(self.handle, *args, **kw)

    def forward(self, *args, **kw):
        return sgb_forward(self.handle, *args, **kw)

    def device_status(self, workspace, stream=None) -> str:
        return sgb_status_string(sgb_device_status(self.handle, workspace, stream))

    def runs_view(self, workspace, num_indices: int, B: int) -> dict:
        return sgb_runs_view_get(self.handle, workspace, num_indices, B)

    def close(self):
        if self.handle:
            sgb_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
