"""CPU oracle for the pooled embedding-bag backward, and the pooled forward it
differentiates (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``sgb_oracle.c`` (plain C loops, fp64 accumulation);
this module only marshals numpy arrays through ctypes.  See that file for the
passages of the pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgb_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED",
          4: "INDEX_OUT_OF_RANGE", 5: "BAD_OFFSETS"}
POOL = {"sum": 0, "mean": 1, "none": 2}
MODE = {"dense": 0, "sgd": 1, "rowwise_adagrad": 2}


def build(force: bool = False, extra_flags: tuple = ()) -> str:
    """Compile sgb_oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    out = _LIB if not extra_flags else os.path.join(
        _HERE, "liboracle_" + "_".join(f.strip("-").replace("=", "") for f in extra_flags) + ".so")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-fno-fast-math", *extra_flags, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("B", ctypes.c_int32), ("N", ctypes.c_int64),
        ("hash_size_cumsum", ctypes.c_void_p), ("D_offsets", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p), ("indices", ctypes.c_void_p),
        ("per_sample_weights", ctypes.c_void_p), ("pooling", ctypes.c_int32),
        ("grad_output", ctypes.c_void_p), ("grad_is_bf16", ctypes.c_int32),
    ]


_libs: dict = {}


def _lib(path: Optional[str] = None):
    path = path or build()
    if path not in _libs:
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(_Problem)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        lib.orc_validate.argtypes = [P]
        lib.orc_linearize.argtypes = [P, vp, vp, vp]
        lib.orc_runs.argtypes = [i64, vp, vp, i64] + [vp] * 9
        lib.orc_row_grads.argtypes = [P, i64, vp, i32, vp, vp]
        lib.orc_update_rows.argtypes = [i32, i32, i64, vp, i32, vp, f32, f32, vp, vp]
        lib.orc_forward.argtypes = [P, vp, vp]
        u32, u64 = ctypes.c_uint32, ctypes.c_uint64
        lib.orc_philox4x32_10.argtypes = [vp, vp, vp]
        lib.orc_philox4x32_10.restype = None
        lib.orc_bf16_round_array.argtypes = [vp, vp, vp, i64]
        lib.orc_bf16_round_array.restype = None
        lib.orc_update_rows_bf16.argtypes = [i32, i64, vp, i32, vp, f32, f32, vp, vp, vp, i32,
                                             u64, u32]
        lib.orc_f16_round_array.argtypes = [vp, vp, vp, i64]
        lib.orc_f16_round_array.restype = None
        lib.orc_f16_widen_array.argtypes = [vp, vp, i64]
        lib.orc_f16_widen_array.restype = None
        lib.orc_update_rows_f16.argtypes = [i32, i64, vp, i32, vp, f32, f32, vp, vp, vp, i32,
                                            u64, u32]
        lib.orc_i8_quantize.argtypes = [vp, i64, i32, vp]
        lib.orc_i8_quantize.restype = None
        lib.orc_i8_dequantize.argtypes = [vp, i64, i32, vp]
        lib.orc_i8_dequantize.restype = None
        lib.orc_update_rows_int8.argtypes = [i32, i64, vp, i32, vp, f32, f32, vp, i32, vp]
        for f in (lib.orc_validate, lib.orc_linearize, lib.orc_runs,
                  lib.orc_row_grads, lib.orc_update_rows, lib.orc_forward,
                  lib.orc_update_rows_bf16, lib.orc_update_rows_int8, lib.orc_update_rows_f16):
            f.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


@dataclass
class Problem:
    """Host-side description of one backward call (numpy arrays).

    grad_output is float32, or uint16 holding bf16 bit patterns (None for
    the forward).  offsets may be None only for nobag ('none' pooling) with
    T == 1.
    """
    T: int
    B: int
    hash_size_cumsum: np.ndarray
    D_offsets: np.ndarray
    offsets: Optional[np.ndarray]
    indices: np.ndarray
    per_sample_weights: Optional[np.ndarray]
    pooling: str
    grad_output: np.ndarray

    def _c(self):
        # keep contiguous copies alive while the struct is in use
        self._keep = [
            np.ascontiguousarray(self.hash_size_cumsum, dtype=np.int64),
            np.ascontiguousarray(self.D_offsets, dtype=np.int32),
            None if self.offsets is None else np.ascontiguousarray(self.offsets, dtype=np.int64),
            np.ascontiguousarray(self.indices, dtype=np.int64),
            None if self.per_sample_weights is None
            else np.ascontiguousarray(self.per_sample_weights, dtype=np.float32),
            None if self.grad_output is None else np.ascontiguousarray(self.grad_output),
        ]
        hsc, doff, off, idx, psw, g = self._keep
        if g is not None and g.dtype not in (np.float32, np.uint16):
            raise TypeError("grad_output must be float32 or uint16 (bf16 bits)")
        return _Problem(int(self.T), int(self.B), int(idx.shape[0]), _ptr(hsc), _ptr(doff),
                        _ptr(off), _ptr(idx), _ptr(psw), POOL[self.pooling], _ptr(g),
                        1 if g is not None and g.dtype == np.uint16 else 0)


def problem_from_inputs(inp) -> Problem:
    """The Problem of a generated batch (any object with the fields of
    ``synth.Inputs``: T, B, hash_size_cumsum, D_offsets, offsets, indices,
    per_sample_weights, grad_output and ``spec.pooling``)."""
    return Problem(T=inp.T, B=inp.B, hash_size_cumsum=inp.hash_size_cumsum,
                   D_offsets=inp.D_offsets, offsets=inp.offsets, indices=inp.indices,
                   per_sample_weights=inp.per_sample_weights, pooling=inp.spec.pooling,
                   grad_output=inp.grad_output)


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(STATUS.get(st, str(st)), what)


class OracleError(RuntimeError):
    def __init__(self, status: str, what: str):
        super().__init__(f"oracle {what}: {status}")
        self.status = status


def validate(p: Problem, lib: Optional[str] = None) -> str:
    c = p._c()
    return STATUS[_lib(lib).orc_validate(ctypes.byref(c))]


def linearize(p: Problem, lib: Optional[str] = None):
    """Per-lookup (linear id, info, coef) in original order."""
    c = p._c()
    n = c.N
    keys = np.zeros(n, np.int64)
    infos = np.zeros(n, np.int64)
    coefs = np.zeros(n, np.float64)
    _check(_lib(lib).orc_linearize(ctypes.byref(c), _ptr(keys), _ptr(infos), _ptr(coefs)),
           "linearize")
    return keys, infos, coefs


def runs(keys: np.ndarray, infos: np.ndarray, thr: int, lib: Optional[str] = None) -> dict:
    """Stable sort + run-length encoding + long-run list."""
    keys = np.ascontiguousarray(keys, np.int64)
    infos = np.ascontiguousarray(infos, np.int64)
    n = keys.shape[0]
    sk, si, sp = (np.zeros(n, np.int64) for _ in range(3))
    uniq, lens = np.zeros(max(n, 1), np.int64), np.zeros(max(n, 1), np.int64)
    cum = np.zeros(n + 1, np.int64)
    longs = np.zeros(max(n, 1), np.int64)
    nr, nl = np.zeros(1, np.int64), np.zeros(1, np.int64)
    _check(_lib(lib).orc_runs(n, _ptr(keys), _ptr(infos), int(thr), _ptr(sk), _ptr(si), _ptr(sp),
                              _ptr(uniq), _ptr(lens), _ptr(cum), _ptr(nr), _ptr(longs), _ptr(nl)),
           "runs")
    U, L = int(nr[0]), int(nl[0])
    return dict(sorted_keys=sk, sorted_infos=si, sorted_pos=sp, unique_ids=uniq[:U],
                run_lengths=lens[:U], cumulative=cum[:U + 1], num_runs=U,
                long_run_ids=longs[:L], num_long=L)


def row_grads(p: Problem, rows: np.ndarray, lib: Optional[str] = None):
    """Aggregated fp64 gradient of each requested linear row id (sorted, distinct).

    Returns (G [nrows, maxD] float64, hits [nrows] int64)."""
    c = p._c()
    rows = np.ascontiguousarray(rows, np.int64)
    doff = np.asarray(p.D_offsets, np.int64)
    ldg = int(np.max(doff[1:] - doff[:-1]))
    G = np.zeros((rows.shape[0], ldg), np.float64)
    hits = np.zeros(rows.shape[0], np.int64)
    _check(_lib(lib).orc_row_grads(ctypes.byref(c), rows.shape[0], _ptr(rows), ldg, _ptr(G),
                                   _ptr(hits)), "row_grads")
    return G, hits


def update_rows(mode: str, G: np.ndarray, D: np.ndarray, rows0: Optional[np.ndarray],
                mom0: Optional[np.ndarray], lr: float = 0.0, eps: float = 0.0,
                accumulate: bool = False, lib: Optional[str] = None):
    """Apply the output step once per row; returns (rows fp32 [n, ldg], mom fp32 [n])."""
    G = np.ascontiguousarray(G, np.float64)
    n, ldg = G.shape
    rows = np.zeros((n, ldg), np.float32) if rows0 is None else \
        np.ascontiguousarray(rows0, np.float32).copy()
    mom = np.zeros(n, np.float32) if mom0 is None else np.ascontiguousarray(mom0, np.float32).copy()
    D = np.ascontiguousarray(D, np.int32)
    _check(_lib(lib).orc_update_rows(MODE[mode], 1 if accumulate else 0, n, _ptr(D), ldg, _ptr(G),
                                     float(lr), float(eps), _ptr(rows), _ptr(mom)), "update_rows")
    return rows, mom


def philox4x32_10(counter, key, lib: Optional[str] = None) -> np.ndarray:
    """One Philox4x32-10 block: four uint32 words from a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(counter, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    _lib(lib).orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def bf16_round(x: np.ndarray, rnd: Optional[np.ndarray] = None,
               lib: Optional[str] = None) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16): nearest even, or stochastic with one
    uint32 random word per element."""
    x = np.ascontiguousarray(x, np.float32).ravel()
    r = None if rnd is None else np.ascontiguousarray(rnd, np.uint32).ravel()
    out = np.zeros(x.size, np.uint16)
    _lib(lib).orc_bf16_round_array(_ptr(x), _ptr(r), _ptr(out), x.size)
    return out


def update_rows_bf16(mode: str, G: np.ndarray, D: np.ndarray, rows0: np.ndarray,
                     mom0: Optional[np.ndarray], row_ids: np.ndarray, lr: float = 0.0,
                     eps: float = 0.0, stochastic: bool = True, seed: int = 0, offset: int = 0,
                     lib: Optional[str] = None):
    """SGD / row-wise Adagrad on bf16 rows (uint16 bit patterns [n, ldg]);
    returns (rows uint16 [n, ldg], mom fp32 [n])."""
    G = np.ascontiguousarray(G, np.float64)
    n, ldg = G.shape
    rows = np.ascontiguousarray(rows0, np.uint16).copy()
    mom = np.zeros(n, np.float32) if mom0 is None else np.ascontiguousarray(mom0, np.float32).copy()
    D = np.ascontiguousarray(D, np.int32)
    ids = np.ascontiguousarray(row_ids, np.int64)
    _check(_lib(lib).orc_update_rows_bf16(MODE[mode], n, _ptr(D), ldg, _ptr(G), float(lr),
                                          float(eps), _ptr(rows), _ptr(mom), _ptr(ids),
                                          1 if stochastic else 0, int(seed) & (2**64 - 1),
                                          int(offset) & 0xFFFFFFFF), "update_rows_bf16")
    return rows, mom


def f16_round(x: np.ndarray, rnd: Optional[np.ndarray] = None,
              lib: Optional[str] = None) -> np.ndarray:
    """fp32 -> binary16 bit patterns (uint16): nearest even, or stochastic
    with one uint32 random word per element."""
    x = np.ascontiguousarray(x, np.float32).ravel()
    r = None if rnd is None else np.ascontiguousarray(rnd, np.uint32).ravel()
    out = np.zeros(x.size, np.uint16)
    _lib(lib).orc_f16_round_array(_ptr(x), _ptr(r), _ptr(out), x.size)
    return out


def f16_widen(h: np.ndarray, lib: Optional[str] = None) -> np.ndarray:
    """binary16 bit patterns -> fp32 (exact)."""
    h = np.ascontiguousarray(h, np.uint16).ravel()
    out = np.zeros(h.size, np.float32)
    _lib(lib).orc_f16_widen_array(_ptr(h), _ptr(out), h.size)
    return out


def update_rows_f16(mode: str, G: np.ndarray, D: np.ndarray, rows0: np.ndarray,
                    mom0: Optional[np.ndarray], row_ids: np.ndarray, lr: float = 0.0,
                    eps: float = 0.0, stochastic: bool = True, seed: int = 0, offset: int = 0,
                    lib: Optional[str] = None):
    """SGD / row-wise Adagrad on fp16 rows (uint16 bit patterns [n, ldg]);
    returns (rows uint16 [n, ldg], mom fp32 [n])."""
    G = np.ascontiguousarray(G, np.float64)
    n, ldg = G.shape
    rows = np.ascontiguousarray(rows0, np.uint16).copy()
    mom = np.zeros(n, np.float32) if mom0 is None else np.ascontiguousarray(mom0, np.float32).copy()
    D = np.ascontiguousarray(D, np.int32)
    ids = np.ascontiguousarray(row_ids, np.int64)
    _check(_lib(lib).orc_update_rows_f16(MODE[mode], n, _ptr(D), ldg, _ptr(G), float(lr),
                                         float(eps), _ptr(rows), _ptr(mom), _ptr(ids),
                                         1 if stochastic else 0, int(seed) & (2**64 - 1),
                                         int(offset) & 0xFFFFFFFF), "update_rows_f16")
    return rows, mom


def i8_quantize(w: np.ndarray, lib: Optional[str] = None) -> np.ndarray:
    """fp32 rows [n, D] -> INT8 rows [n, D + 8] (codes, then fp32 scale and bias)."""
    w = np.ascontiguousarray(w, np.float32)
    n, D = w.shape
    rows = np.zeros((n, D + 8), np.uint8)
    _lib(lib).orc_i8_quantize(_ptr(w), n, D, _ptr(rows))
    return rows


def i8_dequantize(rows: np.ndarray, lib: Optional[str] = None) -> np.ndarray:
    """INT8 rows [n, D + 8] -> fp32 [n, D]."""
    rows = np.ascontiguousarray(rows, np.uint8)
    n, W = rows.shape
    w = np.zeros((n, W - 8), np.float32)
    _lib(lib).orc_i8_dequantize(_ptr(rows), n, W - 8, _ptr(w))
    return w


def update_rows_int8(mode: str, G: np.ndarray, D: np.ndarray, rows0: np.ndarray,
                     mom0: Optional[np.ndarray], lr: float = 0.0, eps: float = 0.0,
                     lib: Optional[str] = None):
    """SGD / row-wise Adagrad on INT8 rows (uint8 [n, ldr], row k's D[k] codes
    then its scale and bias); returns (rows uint8 [n, ldr], mom fp32 [n])."""
    G = np.ascontiguousarray(G, np.float64)
    n, ldg = G.shape
    rows = np.ascontiguousarray(rows0, np.uint8).copy()
    ldr = rows.shape[1]
    mom = np.zeros(n, np.float32) if mom0 is None else np.ascontiguousarray(mom0, np.float32).copy()
    D = np.ascontiguousarray(D, np.int32)
    _check(_lib(lib).orc_update_rows_int8(MODE[mode], n, _ptr(D), ldg, _ptr(G), float(lr),
                                          float(eps), _ptr(rows), ldr, _ptr(mom)),
           "update_rows_int8")
    return rows, mom


def forward(p: Problem, weights: np.ndarray, lib: Optional[str] = None) -> np.ndarray:
    """Pooled forward: [B][D_offsets[T]] (bag) or [N][D] (nobag) float32, from
    the flat float32 weights (table t at sum_{t'<t} E_t' * D_t', row-major)."""
    c = p._c()
    W = np.ascontiguousarray(weights, np.float32)
    doff = np.asarray(p.D_offsets, np.int64)
    if p.pooling == "none":
        out = np.zeros((c.N, int(doff[1] - doff[0])), np.float32)
    else:
        out = np.zeros((int(p.B) if p.offsets is not None else 1, int(doff[-1])), np.float32)
    _check(_lib(lib).orc_forward(ctypes.byref(c), _ptr(W), _ptr(out)), "forward")
    return out

