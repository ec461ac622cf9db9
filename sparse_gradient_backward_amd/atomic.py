"""Python binding of libsgb_atomic.so, the atomic scatter-add backward kept
as a comparison baseline for the deduplicated path (``include/sgb_atomic.h``).

Argument marshalling only: the computation runs in the library's HIP kernel.
Importing this module fails loudly (ImportError) when the library has not
been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SGB_ATOMIC_LIBRARY") or os.path.join(_HERE, "libsgb_atomic.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "sgb_atomic.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python sparse_gradient_backward_amd/build.py` (hipcc, gfx950)")

# bind to torch's HIP runtime (see the package's __init__)
import torch  # noqa: E402

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_lib.sgb_atomic_backward.restype = ctypes.c_int
_lib.sgb_atomic_backward.argtypes = [
    ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P,
    ctypes.c_int32, _P, ctypes.c_int64, _P, ctypes.c_int32, _P, _P, ctypes.c_float,
    ctypes.c_int32, _P]

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "HIP"}
POOLING = {"sum": 0, "mean": 1, "none": 2}
DTYPE = {"f32": 0, "bf16": 1}


def header_functions() -> list:
    """Names of the functions include/sgb_atomic.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(sgb_\w+)\s*\(", text, re.M)))


def _ptr(t):
    return None if t is None else int(t.data_ptr())


def sgb_atomic_backward(T, hash_size_cumsum, D_offsets, table_offsets, max_D, total_elems,
                        pooling, grad_output, grad_dtype, indices, num_indices, offsets, B,
                        per_sample_weights, out, scale, zero_first, stream=None) -> str:
    """The C call with device tensors (or None) for the pointer arguments."""
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = _lib.sgb_atomic_backward(
        int(T), _ptr(hash_size_cumsum), _ptr(D_offsets), _ptr(table_offsets), int(max_D),
        int(total_elems), POOLING[pooling] if isinstance(pooling, str) else int(pooling),
        _ptr(grad_output), DTYPE[grad_dtype] if isinstance(grad_dtype, str) else int(grad_dtype),
        _ptr(indices), int(num_indices), _ptr(offsets), int(B), _ptr(per_sample_weights),
        _ptr(out), float(scale), int(bool(zero_first)), int(s.cuda_stream))
    return STATUS.get(rc, str(rc))


class AtomicTables:
    """Device copies of the table metadata, so that a call passes only the
    batch and the output."""

    def __init__(self, hash_size_cumsum, D_offsets, pooling: str):
        hsc = np.asarray(hash_size_cumsum, np.int64)
        doff = np.asarray(D_offsets, np.int32)
        E, D = np.diff(hsc), np.diff(doff).astype(np.int64)
        woff = np.concatenate([[0], np.cumsum(E * D)]).astype(np.int64)
        self.T = len(hsc) - 1
        self.pooling = pooling
        self.max_D = int(D.max())
        self.total_elems = int(woff[-1])
        self.d_hsc = torch.from_numpy(hsc).cuda()
        self.d_doff = torch.from_numpy(doff).cuda()
        self.d_woff = torch.from_numpy(woff).cuda()

    def backward(self, grad_output, grad_dtype, indices, offsets, B, per_sample_weights, out,
                 scale=1.0, zero_first=False, stream=None) -> str:
        return sgb_atomic_backward(self.T, self.d_hsc, self.d_doff, self.d_woff, self.max_D,
                                   self.total_elems, self.pooling, grad_output, grad_dtype,
                                   indices, indices.numel(), offsets, B, per_sample_weights, out,
                                   scale, zero_first, stream)
