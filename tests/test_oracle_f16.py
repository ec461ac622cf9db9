"""CPU pins of the oracle's fp16 (IEEE binary16) weight rows: the fp32 ->
fp16 roundings (nearest even and stochastic), the exact widening, and the
SGD / row-wise Adagrad update on fp16 rows.  Each is checked against
something other than the oracle itself: numpy's and torch's IEEE fp32 ->
fp16 conversions, exhaustive counts over a stratified set of rounding words,
closed forms and binomial bounds; planted mistakes must fail a pin."""
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _sample(rng):
    """fp32 values over every range binary16 rounds differently: random bit
    patterns of every exponent, the subnormal range, the overflow edge, exact
    ties and near-ties of the dropped 13 bits, signed zeros and infinities."""
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    x = _f32(bits)
    x = x[np.isfinite(x)]
    sub = (rng.random(20000) * 2.0 ** -14).astype(np.float32) * rng.choice([-1, 1], 20000).astype(np.float32)
    tiny = (rng.random(5000) * 2.0 ** -24).astype(np.float32)
    edge = np.float32(65504.0) + (rng.random(5000) * 48).astype(np.float32)
    kept = rng.integers(0x3380, 0x4780, 20000).astype(np.uint32)  # exponents of the normal fp16 range
    ties = _f32(((kept << 13) | 0x1000) & 0x7FFFFFFF)             # dropped bits exactly half
    near = _f32(((kept << 13) | 0x0FFF) & 0x7FFFFFFF)
    sub_ties = np.float32(2.0 ** -24) * (np.arange(1, 2000, dtype=np.float32) + np.float32(0.5))
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, -65520, 2.0 ** -24,
                        2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 6.1e-5, 1e-45, 3.4e38],
                       np.float32)
    return np.concatenate([x, sub, tiny, edge, ties, near, sub_ties, special]).astype(np.float32)


def test_f16_rne_matches_numpy_and_torch(lib=None):
    rng = np.random.default_rng(11)
    x = _sample(rng)
    got = oracle.f16_round(x, lib=lib)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    ref_t = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref_t)
    nan = oracle.f16_round(np.array([np.nan, -np.nan], np.float32), lib=lib)
    assert nan.tolist() == [0x7E00, 0xFE00]


def test_f16_widen_exact(lib=None):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_widen(h, lib=lib)
    ref = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def _neighbours(x):
    """The binary16 values at and above |x| (as numpy float16 bit patterns,
    from numpy's rounding toward zero of the magnitude) and the fraction."""
    a = np.float64(abs(float(x)))
    lo = np.float16(a)
    if float(lo) > a:
        lo = np.nextafter(lo, np.float16(0))
    hi = np.nextafter(lo, np.float16(np.inf))
    return lo, hi


def test_f16_sr_exhaustive_counts(lib=None):
    """Over the 2^16 words j * 2^16, a value rounds its magnitude up exactly
    ceil(f * 2^16) times (f: its fraction of the spacing above the grid point
    below it), to the two neighbours only; where f * 2^16 is a whole number
    (the normal range) the mean of the rounded values is the value itself."""
    rng = np.random.default_rng(12)
    xs = np.concatenate([
        (rng.standard_normal(20) * 100).astype(np.float32),
        (rng.random(6) * 2.0 ** -14).astype(np.float32),       # fp16 subnormals
        np.array([1.0 - 2.0 ** -13, -3.14159, 65000.5, 7e-6, 2.0 ** -25, -1e-7], np.float32)])
    words = np.arange(1 << 16, dtype=np.uint32) << 16
    for x in xs:
        h = oracle.f16_round(np.full(1 << 16, x, np.float32), words, lib=lib)
        lo, hi = _neighbours(x)
        sign = 0x8000 if x < 0 else 0
        lo_b = int(lo.view(np.uint16)) | sign
        hi_b = int(hi.view(np.uint16)) | sign
        assert set(np.unique(h).tolist()) <= {lo_b, hi_b}, x
        u = float(hi) - float(lo)
        f = (abs(float(x)) - float(lo)) / u
        assert int(np.sum(h == hi_b)) == int(np.ceil(f * 65536)), x
        if float(f * 65536).is_integer():
            vals = h.view(np.float16).astype(np.float64)
            assert np.isclose(vals.mean(), float(x), rtol=1e-12, atol=0), x


def test_f16_sr_special_cases(lib=None):
    rng = np.random.default_rng(13)
    words = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    # binary16 values never move
    exact = rng.integers(0, 0x7C00, 20000).astype(np.uint16)
    exact = np.where(rng.random(20000) < 0.5, exact, exact | 0x8000).astype(np.uint16)
    xf = exact.view(np.float16).astype(np.float32)
    assert np.array_equal(oracle.f16_round(xf, words, lib=lib), exact)
    # sign symmetry
    x = (rng.standard_normal(20000) * 10).astype(np.float32)
    a = oracle.f16_round(x, words, lib=lib)
    b = oracle.f16_round(-x, words, lib=lib)
    assert np.array_equal(a ^ b, np.full_like(a, 0x8000))
    # word 0 always rounds a non-grid magnitude up, the largest word down
    y = np.array([1.0 + 2.0 ** -12, 65519.0, 3e-8], np.float32)
    up = oracle.f16_round(y, np.zeros(3, np.uint32), lib=lib)
    dn = oracle.f16_round(y, np.full(3, 2**32 - 1, np.uint32), lib=lib)
    assert up.tolist() == [0x3C01, 0x7C00, 0x0001]
    assert dn.tolist() == [0x3C00, 0x7BFF, 0x0000]
    # non-finite
    nf = oracle.f16_round(np.array([np.inf, -np.inf, np.nan], np.float32),
                          np.array([0, 2**32 - 1, 5], np.uint32), lib=lib)
    assert nf.tolist() == [0x7C00, 0xFC00, 0x7E00]


def test_f16_sgd_rne_closed_form(lib=None):
    """w0 = 1, G = 2^-13, lr = 1: the fp32 result 1 - 2^-13 lies a quarter of
    the spacing below 1 (2^-11 in [0.5, 1)), so nearest even gives 1 exactly;
    lr = 3 puts it three quarters below: 1 - 2^-11 (0x3BFF)."""
    n = 4
    G = np.full((n, 8), 2.0 ** -13)
    rows = np.full((n, 8), 0x3C00, np.uint16)
    D = np.full(n, 8)
    out, _ = oracle.update_rows_f16("sgd", G, D, rows, None, np.arange(n), lr=1.0,
                                    stochastic=False, lib=lib)
    assert np.all(out == 0x3C00)
    out, _ = oracle.update_rows_f16("sgd", G, D, rows, None, np.arange(n), lr=3.0,
                                    stochastic=False, lib=lib)
    assert np.all(out == 0x3BFF)


def test_f16_sgd_sr_rate(lib=None):
    """The quarter-spacing step with stochastic rounding over 4096 rows of 16
    columns: the fraction rounded down to 0x3BFF is 1/4 within binomial bounds
    (5 sigma); the same seed, offset and rows give the same result; each
    element follows its own Philox word (up iff word < 0.75 * 2^32)."""
    n, D = 4096, 16
    G = np.full((n, D), 2.0 ** -13)
    rows = np.full((n, D), 0x3C00, np.uint16)
    ids = np.arange(n, dtype=np.int64) * 7919 + 3
    out, _ = oracle.update_rows_f16("sgd", G, np.full(n, D), rows, None, ids, lr=1.0,
                                    stochastic=True, seed=4321, offset=5, lib=lib)
    assert set(np.unique(out).tolist()) <= {0x3C00, 0x3BFF}
    k = int(np.sum(out == 0x3BFF))
    mean, sd = n * D / 4, np.sqrt(n * D * 0.25 * 0.75)
    assert abs(k - mean) < 5 * sd
    again, _ = oracle.update_rows_f16("sgd", G, np.full(n, D), rows, None, ids, lr=1.0,
                                      stochastic=True, seed=4321, offset=5, lib=lib)
    assert np.array_equal(out, again)
    for r in (0, 9, 4095):
        for c in (0, 2, 7, 15):
            w = int(oracle.philox4x32_10((c // 4, ids[r] & 0xFFFFFFFF, ids[r] >> 32, 5),
                                         (4321, 0), lib=lib)[c % 4])
            assert out[r, c] == (0x3C00 if w < 0.75 * 2**32 else 0x3BFF)


def test_f16_adagrad_closed_form(lib=None):
    """m0 = 0, one lookup: w = w0 - lr * g / (rms(g) + eps), the fp32 value
    rounded to nearest even fp16 (numpy's conversion); state = mean(g^2)."""
    rng = np.random.default_rng(14)
    n, D = 50, 24
    g = rng.standard_normal((n, D))
    w0 = (rng.standard_normal((n, D)) * 0.01).astype(np.float16)
    rows = w0.view(np.uint16)
    lr, eps = 0.01, 1e-8
    out, mom = oracle.update_rows_f16("rowwise_adagrad", g, np.full(n, D), rows,
                                      np.zeros(n, np.float32), np.arange(n), lr=lr, eps=eps,
                                      stochastic=False, lib=lib)
    rms = np.sqrt((g * g).mean(axis=1))
    exp32 = (w0.astype(np.float64) - lr * g / (rms[:, None] + eps)).astype(np.float32)
    assert np.array_equal(out, exp32.astype(np.float16).view(np.uint16))
    assert np.allclose(mom, (g * g).mean(axis=1), rtol=1e-6)


_PINS = [test_f16_rne_matches_numpy_and_torch, test_f16_widen_exact,
         test_f16_sr_exhaustive_counts, test_f16_sr_special_cases, test_f16_sgd_rne_closed_form,
         test_f16_sgd_sr_rate, test_f16_adagrad_closed_form]

_MUTANTS = [
    ("subnormal spacing 2^-23", r"\*u = ldexp\(1\.0, -24\);", "*u = ldexp(1.0, -23);"),
    ("ties away from zero", r"\(f == 0\.5 && fmod\(q, 2\.0\) == 1\.0\)", "(f == 0.5)"),
    ("mantissa of 9 bits", r"\*u = ldexp\(1\.0, k - 1 - 10\);", "*u = ldexp(1.0, k - 1 - 9);"),
    ("overflow saturates", r"if \(v > 65504\.0\) return \(uint16_t\)\(s \| 0x7C00u\);",
     "if (v > 65504.0) return (uint16_t)(s | 0x7BFFu);"),
    ("sr compares with <=", r"if \(\(double\)rnd < f \* 4294967296\.0\) q \+= 1\.0;",
     "if ((double)rnd <= f * 4294967296.0) q += 1.0;"),
    ("sr uses 16 bits", r"if \(\(double\)rnd < f \* 4294967296\.0\) q \+= 1\.0;",
     "if ((double)(rnd & 0xFFFFu) < f * 65536.0) q += 1.0;"),
    ("sr down-biased", r"if \(\(double\)rnd < f \* 4294967296\.0\) q \+= 1\.0;",
     "if ((double)rnd < f * 2147483648.0) q += 1.0;"),
    ("nan not quiet", r"\| 0x7E00u\);", "| 0x7C01u);"),
    ("widening subnormal wrong", r"else if \(ex == 0\) v = ldexp\(\(double\)man, -24\);",
     "else if (ex == 0) v = ldexp((double)man, -23);"),
    ("f16 rows rounded nearest even under SR",
     r"h\[d\] = stochastic \? orc_f16_sr\(tmp\[d\], orc_sr_word\(seed, offset, row_ids\[k\], d\)\)",
     "h[d] = 0 ? orc_f16_sr(tmp[d], orc_sr_word(seed, offset, row_ids[k], d))"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("desc,pattern,repl", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_planted_mistakes_f16(desc, pattern, repl):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "sgb_oracle.c")).read()
    new, n = re.subn(pattern, repl, src)
    assert n >= 1, f"mutant '{desc}' did not apply"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "m.c")
        open(path, "w").write(new)
        lib = os.path.join(tmp, f"lib_{abs(hash(desc))}.so")
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", path, "-o", lib, "-lm"])
        caught = 0
        for pin in _PINS:
            try:
                pin(lib=lib)
            except Exception:
                caught += 1
        assert caught > 0, f"no pin catches: {desc}"
