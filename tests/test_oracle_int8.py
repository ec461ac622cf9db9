"""CPU pins of the oracle's INT8 row-wise quantized weight rows: the
quantization of a row (codes and per-row scale / bias stored after the
codes), its inverse, and SGD / row-wise Adagrad on quantized rows.  Pinned by
hand-derived rows, invariants any correct row-wise min/max quantizer meets,
closed forms of the updates, and planted mistakes that must fail a pin."""
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle


def _qp(rows):
    D = rows.shape[1] - 8
    qp = np.ascontiguousarray(rows[:, D:]).view(np.float32)
    return rows[:, :D], qp[:, 0], qp[:, 1]


def test_hand_row(lib=None):
    """[0, 1, 0.5, 0.25]: bias 0, scale fl(1/255); 0.5 / fl(1/255) = 127.49998
    -> 127, 0.25 / fl(1/255) = 63.74999 -> 64; the pair follows the codes."""
    rows = oracle.i8_quantize(np.array([[0.0, 1.0, 0.5, 0.25]], np.float32), lib=lib)
    codes, scale, bias = _qp(rows)
    assert codes.tolist() == [[0, 255, 127, 64]]
    assert scale[0] == np.float32(1.0) / np.float32(255.0) and bias[0] == 0.0
    w = oracle.i8_dequantize(rows, lib=lib)
    assert w[0, 0] == 0.0 and abs(w[0, 1] - 1.0) < 1e-7
    # a row from -3 to 5: bias -3, scale fl(8/255), which lies above 8/255, so
    # 1 -> 4 / fl(8/255) = 127.49999 -> 127; the ends map to 0 and 255
    rows = oracle.i8_quantize(np.array([[5.0, -3.0, 1.0, -3.0]], np.float32), lib=lib)
    codes, scale, bias = _qp(rows)
    assert codes.tolist() == [[255, 0, 127, 0]] and bias[0] == -3.0
    assert scale[0] == np.float32(8.0) / np.float32(255.0)


def test_quantize_invariants(lib=None):
    rng = np.random.default_rng(7)
    for D in (4, 16, 132, 1024):
        w = (rng.standard_normal((40, D)) * rng.uniform(1e-3, 10, (40, 1))).astype(np.float32)
        rows = oracle.i8_quantize(w, lib=lib)
        codes, scale, bias = _qp(rows)
        assert np.array_equal(bias, w.min(axis=1))
        assert np.array_equal(scale, (w.max(axis=1) - w.min(axis=1)) / np.float32(255.0))
        # the row's minimum gets code 0, its maximum 255
        assert np.all(codes[np.arange(40), w.argmin(axis=1)] == 0)
        assert np.all(codes[np.arange(40), w.argmax(axis=1)] == 255)
        # every value is within half a step (plus fp32 rounding) of its code's value
        back = oracle.i8_dequantize(rows, lib=lib)
        assert np.all(np.abs(back - w) <= scale[:, None] * 0.5001 + 1e-6 * np.abs(w))
        # codes are monotone in the values
        for k in range(5):
            o = np.argsort(w[k], kind="stable")
            assert np.all(np.diff(codes[k][o].astype(int)) >= 0)


def test_constant_row(lib=None):
    rows = oracle.i8_quantize(np.full((3, 8), 0.75, np.float32), lib=lib)
    codes, scale, bias = _qp(rows)
    assert np.all(codes == 0) and np.all(scale == 0) and np.all(bias == 0.75)
    assert np.all(oracle.i8_dequantize(rows, lib=lib) == 0.75)


def _rows(rng, n, D):
    w = (rng.standard_normal((n, D)) * 0.01).astype(np.float32)
    return oracle.i8_quantize(w, lib=None)


def test_sgd_zero_and_uniform_steps(lib=None):
    """G = 0 leaves every code and the parameters as they are (to one fp32 ulp);
    a constant G row shifts the bias by -lr*g and keeps the codes."""
    rng = np.random.default_rng(8)
    n, D = 30, 64
    rows0 = _rows(rng, n, D)
    out, _ = oracle.update_rows_int8("sgd", np.zeros((n, D)), np.full(n, D), rows0, None, lr=0.1,
                                     lib=lib)
    c0, s0, b0 = _qp(rows0)
    c1, s1, b1 = _qp(out)
    assert np.array_equal(c0, c1) and np.array_equal(b0, b1)
    assert np.allclose(s1, s0, rtol=2e-7, atol=0)
    g = rng.uniform(-1, 1, n)
    out, _ = oracle.update_rows_int8("sgd", np.repeat(g[:, None], D, axis=1), np.full(n, D), rows0,
                                     None, lr=0.01, lib=lib)
    c2, s2, b2 = _qp(out)
    assert np.array_equal(c0, c2)
    assert np.allclose(b2, b0 - 0.01 * g, rtol=0, atol=1e-7)
    assert np.allclose(s2, s0, rtol=1e-4, atol=0)


def test_adagrad_closed_form(lib=None):
    """m0 = 0, one lookup: w' = w - lr * g / (rms(g) + eps) from the dequantized
    row, then the row is quantized again; state = mean(g^2)."""
    rng = np.random.default_rng(9)
    n, D = 25, 32
    rows0 = _rows(rng, n, D)
    g = rng.standard_normal((n, D))
    lr, eps = 0.01, 1e-8
    out, mom = oracle.update_rows_int8("rowwise_adagrad", g, np.full(n, D), rows0,
                                       np.zeros(n, np.float32), lr=lr, eps=eps, lib=lib)
    w0 = oracle.i8_dequantize(rows0, lib=lib).astype(np.float64)
    rms = np.sqrt((g * g).mean(axis=1))
    exp = (w0 - lr * g / (rms[:, None] + eps)).astype(np.float32)
    ref = oracle.i8_quantize(exp, lib=lib)
    # the closed form rounds in another order: an fp32 value may move by an
    # ulp and flip a code that sits on .5, nothing more
    c, s, b = _qp(out)
    rc, rs, rb = _qp(ref)
    assert np.allclose(b, rb, rtol=1e-6, atol=0) and np.allclose(s, rs, rtol=1e-5, atol=0)
    d = np.abs(c.astype(int) - rc.astype(int))
    assert d.max() <= 1 and (d > 0).mean() < 0.02
    assert np.allclose(mom, (g * g).mean(axis=1), rtol=1e-6)


def test_rows_wider_than_their_table(lib=None):
    """Rows of several widths share one buffer of ldr bytes per row; bytes past
    D + 8 are left alone."""
    rng = np.random.default_rng(10)
    D = np.array([8, 16, 4])
    ldr = 16 + 8 + 4
    rows = np.full((3, ldr), 0xAB, np.uint8)
    for k, d in enumerate(D):
        rows[k, :d + 8] = _rows(rng, 1, d)[0]
    out, _ = oracle.update_rows_int8("sgd", rng.standard_normal((3, 16)), D, rows, None, lr=0.05,
                                     lib=lib)
    for k, d in enumerate(D):
        assert np.all(out[k, d + 8:] == 0xAB)
        w0 = oracle.i8_dequantize(rows[k:k + 1, :d + 8], lib=lib)
        w1 = oracle.i8_dequantize(out[k:k + 1, :d + 8], lib=lib)
        assert not np.array_equal(w0, w1)


_PINS = [test_hand_row, test_quantize_invariants, test_constant_row,
         test_sgd_zero_and_uniform_steps, test_adagrad_closed_form, test_rows_wider_than_their_table]

_MUTANTS = [
    ("scale over 256", r"\(mx - mn\) / 255\.0f", "(mx - mn) / 256.0f"),
    ("bias is the max", r"const float bias = mn;", "const float bias = mx;"),
    ("codes truncated", r"rintf\(\(w\[d\] - bias\) / scale\)", "truncf((w[d] - bias) / scale)"),
    ("bias not subtracted", r"rintf\(\(w\[d\] - bias\) / scale\)", "rintf(w[d] / scale)"),
    ("parameters swapped", r"memcpy\(row \+ D, &scale, 4\);", "memcpy(row + D, &bias, 4); (void)scale;"),
    ("dequantize without bias", r"return fmaf\(\(float\)c, scale, bias\);", "return (float)c * scale;"),
    ("update skipped", r"if \(st == ORC_OK\) orc_i8_quantize_row\(tmp, Dk, r\);",
     "if (st == ORC_OK) { orc_i8_dequantize(r, 1, Dk, tmp); orc_i8_quantize_row(tmp, Dk, r); }"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("desc,pattern,repl", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_planted_mistakes_int8(desc, pattern, repl):
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
