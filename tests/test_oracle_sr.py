"""CPU pins of the oracle's bf16 weight rows: the Philox4x32-10 generator, the
fp32 -> bf16 roundings (nearest even and stochastic) and the SGD / row-wise
Adagrad update on bf16 rows.  Each is checked against something other than
the oracle itself: the generator's published known-answer vectors, torch's
fp32 -> bf16 conversion, exhaustive counts over all 2^16 rounding words,
closed forms, and binomial bounds; planted mistakes must fail a pin."""
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle

# Known-answer vectors of Philox4x32-10 published with the generator
# (Salmon et al., SC'11; the Random123 distribution's kat_vectors):
# (counter, key, output)
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def test_philox_known_answers(lib=None):
    for ctr, key, out in KAT:
        assert tuple(int(v) for v in oracle.philox4x32_10(ctr, key, lib=lib)) == out


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def test_rne_matches_torch(lib=None):
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * (10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32),
        # exact ties (low half 0x8000) with even and odd kept halves, and near-ties
        (((rng.integers(0, 2**15, 4000).astype(np.uint32) << 16) | 0x8000)).view(np.float32),
        (((rng.integers(0, 2**15, 4000).astype(np.uint32) << 16) | 0x7FFF)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -1e-40, 1e-45], np.float32)])
    x = x[~np.isnan(x)]   # NaNs: checked below
    got = oracle.bf16_round(x, lib=lib)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = oracle.bf16_round(np.array([np.nan, -np.nan], np.float32), lib=lib)
    assert np.all(np.isnan(torch.from_numpy(nan.view(np.int16)).view(torch.bfloat16).float().numpy()))


def test_sr_exhaustive_roundup_count(lib=None):
    """Over all 2^16 rounding words, a value rounds its magnitude up exactly
    (dropped low 16 bits) times and down otherwise: the mean of the rounded
    values is the value itself (unbiased)."""
    rng = np.random.default_rng(4)
    xs = rng.standard_normal(24).astype(np.float32) * np.float32(1e3)
    xs = np.concatenate([xs, np.array([1.0, -2.5, 1e-30, -7.0e20], np.float32)])
    words = (np.arange(1 << 16, dtype=np.uint32) << 16)
    for x in xs:
        u = int(_bits(x))
        h = oracle.bf16_round(np.full(1 << 16, x, np.float32), words, lib=lib)
        down, up = u >> 16, (u >> 16) + 1
        assert set(np.unique(h).tolist()) <= {down, up}
        assert int(np.sum(h == up)) == (u & 0xFFFF)
        vals = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.isclose(vals.mean(), float(x), rtol=1e-12, atol=0)


def test_sr_special_cases(lib=None):
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2**32, 5000, dtype=np.uint64).astype(np.uint32)
    # values representable in bf16 never move
    exact = ((rng.integers(0, 2**16, 5000).astype(np.uint32) << 16)).view(np.float32)
    exact = np.where(np.isfinite(exact), exact, np.float32(1.0)).astype(np.float32)
    assert np.array_equal(oracle.bf16_round(exact, words, lib=lib), (_bits(exact) >> 16).astype(np.uint16))
    x = rng.standard_normal(5000).astype(np.float32)
    # a zero word truncates; sign symmetry
    assert np.array_equal(oracle.bf16_round(x, np.zeros(5000, np.uint32), lib=lib),
                          (_bits(x) >> 16).astype(np.uint16))
    assert np.array_equal(oracle.bf16_round(-x, words, lib=lib),
                          oracle.bf16_round(x, words, lib=lib) ^ np.uint16(0x8000))
    inf = oracle.bf16_round(np.array([np.inf, -np.inf], np.float32), np.array([2**32 - 1] * 2, np.uint32), lib=lib)
    assert inf.tolist() == [0x7F80, 0xFF80]


def test_bf16_sgd_rne_closed_form(lib=None):
    """w0 = 1 (bf16), G = 2^-10, lr = 1: the fp32 result 1 - 2^-10 lies a
    quarter ulp below 1.0, so nearest even gives 1.0 exactly; with lr = 3 the
    result 1 - 3 * 2^-10 is three quarters of an ulp below: 1 - 2^-8."""
    n = 4
    G = np.full((n, 8), 2.0 ** -10)
    rows = np.full((n, 8), 0x3F80, np.uint16)
    D = np.full(n, 8)
    out, _ = oracle.update_rows_bf16("sgd", G, D, rows, None, np.arange(n), lr=1.0,
                                     stochastic=False, lib=lib)
    assert np.all(out == 0x3F80)
    out, _ = oracle.update_rows_bf16("sgd", G, D, rows, None, np.arange(n), lr=3.0,
                                     stochastic=False, lib=lib)
    assert np.all(out == 0x3F7F)


def test_bf16_sgd_sr_rate(lib=None):
    """Same quarter-ulp step with stochastic rounding over 4096 rows of 16
    columns: the fraction rounded down to 1 - 2^-8 is 1/4 within binomial
    bounds (5 sigma), and the result depends on seed, offset and row only."""
    n, D = 4096, 16
    G = np.full((n, D), 2.0 ** -10)
    rows = np.full((n, D), 0x3F80, np.uint16)
    ids = np.arange(n, dtype=np.int64) * 7919 + 3
    out, _ = oracle.update_rows_bf16("sgd", G, np.full(n, D), rows, None, ids, lr=1.0,
                                     stochastic=True, seed=1234, offset=9, lib=lib)
    assert set(np.unique(out).tolist()) <= {0x3F80, 0x3F7F}
    k = int(np.sum(out == 0x3F7F))
    mean, sd = n * D / 4, np.sqrt(n * D * 0.25 * 0.75)
    assert abs(k - mean) < 5 * sd
    again, _ = oracle.update_rows_bf16("sgd", G, np.full(n, D), rows, None, ids, lr=1.0,
                                       stochastic=True, seed=1234, offset=9, lib=lib)
    assert np.array_equal(out, again)
    other, _ = oracle.update_rows_bf16("sgd", G, np.full(n, D), rows, None, ids, lr=1.0,
                                       stochastic=True, seed=1235, offset=9, lib=lib)
    assert not np.array_equal(out, other)
    # element (row, col) takes word col % 4 of the Philox block (col // 4, row, 0, offset)
    for r in (0, 5, 4095):
        for c in (0, 3, 6, 15):
            w = oracle.philox4x32_10((c // 4, ids[r] & 0xFFFFFFFF, ids[r] >> 32, 9),
                                     (1234, 0), lib=lib)[c % 4]
            exp = 0x3F7F if (0x3F7FC000 + (int(w) >> 16)) >> 16 == 0x3F7F else 0x3F80
            assert out[r, c] == exp


def test_bf16_adagrad_closed_form(lib=None):
    """m0 = 0, one lookup: w = w0 - lr * g / (rms(g) + eps), the fp32 value
    rounded to nearest even bf16 (torch's conversion); state = mean(g^2)."""
    rng = np.random.default_rng(6)
    n, D = 50, 24
    g = rng.standard_normal((n, D))
    w0 = torch.from_numpy(rng.standard_normal((n, D)).astype(np.float32) * 0.01).to(torch.bfloat16)
    rows = w0.view(torch.int16).numpy().view(np.uint16)
    lr, eps = 0.01, 1e-8
    out, mom = oracle.update_rows_bf16("rowwise_adagrad", g, np.full(n, D), rows,
                                       np.zeros(n, np.float32), np.arange(n), lr=lr, eps=eps,
                                       stochastic=False, lib=lib)
    rms = np.sqrt((g * g).mean(axis=1))
    exp32 = (w0.float().numpy().astype(np.float64) - lr * g / (rms[:, None] + eps)).astype(np.float32)
    ref = torch.from_numpy(exp32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)
    assert np.allclose(mom, (g * g).mean(axis=1), rtol=1e-6)


_PINS = [test_philox_known_answers, test_rne_matches_torch, test_sr_exhaustive_roundup_count,
         test_sr_special_cases, test_bf16_sgd_rne_closed_form, test_bf16_sgd_sr_rate,
         test_bf16_adagrad_closed_form]

_MUTANTS = [
    ("philox key bump missing", r"k0 \+= 0x9E3779B9u;", ""),
    ("philox multiplier swapped", r"0xCD9E8D57u \* c2, hi1 = orc_mulhi32\(0xCD9E8D57u, c2\)",
     "0xD2511F53u * c2, hi1 = orc_mulhi32(0xD2511F53u, c2)"),
    ("philox 9 rounds", r"round < 10;", "round < 9;"),
    ("rne tie to even dropped", r"\(u \+ 0x7FFFu \+ \(\(u >> 16\) & 1u\)\) >> 16",
     "(u + 0x8000u) >> 16"),
    ("sr uses low bits", r"\(u \+ \(rnd >> 16\)\) >> 16", "(u + (rnd & 0xFFFFu)) >> 16"),
    ("sr off by one", r"\(u \+ \(rnd >> 16\)\) >> 16", "(u + (rnd >> 16) + 1u) >> 16"),
    ("sr word from wrong column", r"return out\[col & 3\];", "return out[0];"),
    ("sr counter without offset", r"\(uint32_t\)\(\(uint64_t\)row >> 32\), offset\}",
     "(uint32_t)((uint64_t)row >> 32), 0u}"),
    ("bf16 rows widened wrong", r"const uint32_t u = \(\(uint32_t\)h\[d\]\) << 16;",
     "const uint32_t u = ((uint32_t)h[d]) << 15;"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("desc,pattern,repl", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_planted_mistakes_bf16(desc, pattern, repl):
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
