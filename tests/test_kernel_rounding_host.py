"""The kernels' 16-bit rounding and widening helpers, compiled for the host
and compared bit for bit with the oracle's (CPU, no GPU needed).

The device functions bf16_rne, bf16_sr, f16_widen and f16_round are taken
from kernels.hip as written (the HIP-only qualifiers and bit casts are
defined for the host) and built with g++ into a small library.  f16_widen is
compared on all 65 536 binary16 patterns (NaNs as NaNs); the roundings on
fp32 values of every range binary16 and bf16 round differently (random
patterns of every exponent, the subnormal grid, the overflow edge, exact
ties and near-ties of the dropped bits, signed zeros, infinities and NaNs)
and, for the normal binary16 range, on a stride through every exponent and
significand, each value with several rounding words, including the words
that sit exactly at the stochastic-rounding threshold.  The GPU tests compare rows after a whole
update, within a rounding; these pin the rounding itself exactly.
"""
import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
KERNELS = os.path.join(HERE, "..", "sparse_gradient_backward_amd", "csrc", "kernels.hip")

HELPERS = ["bf16_nonfinite", "bf16_rne", "bf16_sr", "f16_widen", "f16_round"]

PRELUDE = r"""
#include <cstdint>
#include <cstring>
#include <cstddef>
#define __device__
#define __forceinline__ inline
static inline uint32_t __float_as_uint(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static inline float __uint_as_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
"""

WRAPPERS = r"""
extern "C" {
void k_bf16_round_array(const float* x, const uint32_t* rnd, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i)
    out[i] = (uint16_t)(rnd ? bf16_sr(x[i], rnd[i]) : bf16_rne(x[i]));
}
void k_f16_round_array(const float* x, const uint32_t* rnd, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i)
    out[i] = (uint16_t)(rnd ? f16_round(x[i], rnd[i], true) : f16_round(x[i], 0u, false));
}
void k_f16_widen_array(const uint16_t* h, float* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = f16_widen(h[i]);
}
}
"""


def _extract(src, name):
    """The text of device function `name` (its signature line through the
    matching closing brace)."""
    m = re.search(r"__device__ __forceinline__ \w+ " + name + r"\(", src)
    assert m, f"{name} not found in kernels.hip"
    i = src.index("{", m.end())
    depth = 0
    for j in range(i, len(src)):
        if src[j] == "{":
            depth += 1
        elif src[j] == "}":
            depth -= 1
            if depth == 0:
                return src[m.start():j + 1]
    raise AssertionError(f"unbalanced braces in {name}")


@pytest.fixture(scope="module")
def klib():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    src = open(KERNELS).read()
    body = PRELUDE + "\n".join(_extract(src, n) for n in HELPERS) + WRAPPERS
    d = tempfile.mkdtemp(prefix="sgb_round_")
    cpp, so = os.path.join(d, "r.cpp"), os.path.join(d, "r.so")
    open(cpp, "w").write(body)
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", cpp, "-o", so], check=True)
    lib = ctypes.CDLL(so)
    yield lib
    shutil.rmtree(d, ignore_errors=True)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _kround(lib, fn, x, rnd):
    x = np.ascontiguousarray(x, np.float32)
    out = np.zeros(x.size, np.uint16)
    r = None if rnd is None else np.ascontiguousarray(rnd, np.uint32)
    getattr(lib, fn)(_p(x), None if r is None else _p(r), _p(out), ctypes.c_size_t(x.size))
    return out


def _values(rng, top_kept):
    """fp32 values over every range the 16-bit formats round differently."""
    bits = rng.integers(0, 2**32, 400000, dtype=np.uint64).astype(np.uint32)
    kept = rng.integers(0, top_kept, 40000).astype(np.uint32)
    nan = np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0xFF812345], np.uint32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, -65520, 2.0 ** -24,
                        2.0 ** -25, 2.0 ** -14, 6.1e-5, 1e-45, 3.4e38, -3.4e38], np.float32)
    sub = (rng.random(20000) * 2.0 ** -14).astype(np.float32)
    return np.concatenate([bits.view(np.float32), sub, -sub, special, nan.view(np.float32),
                           ((kept << 13) | 0x1000).view(np.float32),     # binary16 ties
                           ((kept << 13) | 0x0FFF).view(np.float32),
                           ((kept << 16) | 0x8000).view(np.float32),     # bf16 ties
                           ((kept << 16) | 0x7FFF).view(np.float32)])


def _words(rng, x, shift):
    """Rounding words: random, all ones, zero, and the words at and just
    below the stochastic threshold of the dropped `shift` bits."""
    u = x.view(np.uint32)
    rem = (u & ((1 << shift) - 1)).astype(np.uint64)
    at = ((rem << (32 - shift)) & 0xFFFFFFFF).astype(np.uint32)
    return [rng.integers(0, 2**32, x.size, dtype=np.uint64).astype(np.uint32),
            np.full(x.size, 0xFFFFFFFF, np.uint32), np.zeros(x.size, np.uint32),
            at, (at.astype(np.int64) - 1).astype(np.uint32)]


def test_f16_widen_all_patterns(klib):
    """Bit-exact on every non-NaN pattern; a NaN widens to a NaN (the kernel
    keeps the payload, the oracle returns the default NaN: no payload
    survives the update, whose rounding makes every NaN 0x7E00)."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out = np.zeros(h.size, np.float32)
    klib.k_f16_widen_array(_p(h), _p(out), ctypes.c_size_t(h.size))
    ref = oracle.f16_widen(h)
    nan = ((h >> 10) & 31) == 31
    nan &= (h & 1023) != 0
    assert np.array_equal(out.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.isnan(out[nan]).all() and np.isnan(ref[nan]).all()


def test_f16_round_matches_oracle(klib):
    rng = np.random.default_rng(7)
    x = _values(rng, 1 << 18)
    assert np.array_equal(_kround(klib, "k_f16_round_array", x, None), oracle.f16_round(x))
    for w in _words(rng, x, 13):
        assert np.array_equal(_kround(klib, "k_f16_round_array", x, w), oracle.f16_round(x, w))


def test_f16_round_normal_range_stride(klib):
    """Every binade of the normal binary16 range (2^-14 .. 2^16) and beyond
    its edges, a stride through the significands, both signs."""
    rng = np.random.default_rng(11)
    u = np.arange(0x38000000, 0x48000000, 997, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([u, u | 0x80000000]).view(np.float32)
    assert np.array_equal(_kround(klib, "k_f16_round_array", x, None), oracle.f16_round(x))
    for w in _words(rng, x, 13):
        assert np.array_equal(_kround(klib, "k_f16_round_array", x, w), oracle.f16_round(x, w))


def test_bf16_round_matches_oracle(klib):
    rng = np.random.default_rng(13)
    x = _values(rng, 1 << 15)
    assert np.array_equal(_kround(klib, "k_bf16_round_array", x, None), oracle.bf16_round(x))
    for w in _words(rng, x, 16):
        assert np.array_equal(_kround(klib, "k_bf16_round_array", x, w), oracle.bf16_round(x, w))
