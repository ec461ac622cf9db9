"""Pins of the oracle's pooled forward against things other than itself (CPU only).

The forward is pinned by a hand-worked case, by torch's own embedding_bag /
embedding in fp64, by its adjointness to the backward oracle's dense
gradient (itself pinned in test_oracle.py), and by empty-bag and error
cases; planted mistakes in a copy of the oracle source must each fail a pin.
"""
import json
import os
import re
import shutil
import subprocess
import tempfile
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "hand_forward_two_tables.json")) as f:
        g = json.load(f)
    p = oracle.Problem(T=g["T"], B=g["B"], hash_size_cumsum=np.array(g["hash_size_cumsum"]),
                       D_offsets=np.array(g["D_offsets"]), offsets=np.array(g["offsets"]),
                       indices=np.array(g["indices"]),
                       per_sample_weights=np.array(g["per_sample_weights"], np.float32),
                       pooling="sum", grad_output=None)
    return g, p, np.array(g["weights"], np.float32)


def _problem(inp, grad=False):
    return oracle.Problem(T=inp.T, B=inp.B, hash_size_cumsum=inp.hash_size_cumsum,
                          D_offsets=inp.D_offsets, offsets=inp.offsets, indices=inp.indices,
                          per_sample_weights=inp.per_sample_weights, pooling=inp.spec.pooling,
                          grad_output=inp.grad_output if grad else None)


def _small(seed, T=3, E=(7, 5, 11), D=(4, 12, 8), B=6, lens=("uniform", 0, 5), pooling="sum",
           weighted=False):
    s = synth.Spec("small", T, tuple(E), tuple(D), B, lens, ("uniform",), pooling, weighted,
                   "f32", "dense", seed=seed)
    return synth.generate(s)


def _weights(inp, seed):
    return np.random.default_rng(seed).standard_normal(int(inp.weights_offsets[-1])).astype(np.float32)


def test_forward_hand_golden(lib=None):
    g, p, W = _golden()
    out = oracle.forward(p, W, lib=lib)
    np.testing.assert_array_equal(out, np.array(g["expected_sum_weighted"], np.float32))
    out = oracle.forward(replace(p, pooling="mean", per_sample_weights=None), W, lib=lib)
    np.testing.assert_array_equal(out, np.array(g["expected_mean"], np.float64).astype(np.float32))


@pytest.mark.parametrize("pooling,weighted", [("sum", False), ("sum", True), ("mean", False)])
@pytest.mark.parametrize("seed", [1, 2])
def test_forward_against_torch_embedding_bag(pooling, weighted, seed, lib=None):
    inp = _small(seed, pooling=pooling, weighted=weighted)
    W = _weights(inp, seed)
    out = oracle.forward(_problem(inp), W, lib=lib)
    for t in range(inp.T):
        E = int(inp.hash_size_cumsum[t + 1] - inp.hash_size_cumsum[t])
        D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
        w0 = int(inp.weights_offsets[t])
        w = torch.from_numpy(W[w0:w0 + E * D].astype(np.float64).reshape(E, D))
        off = inp.offsets[t * inp.B:(t + 1) * inp.B + 1]
        idx = torch.from_numpy(inp.indices[off[0]:off[-1]])
        psw = None
        if inp.per_sample_weights is not None:
            psw = torch.from_numpy(inp.per_sample_weights[off[0]:off[-1]].astype(np.float64))
        ref = torch.nn.functional.embedding_bag(idx, w, torch.from_numpy(off[:-1] - off[0]),
                                                mode=pooling, per_sample_weights=psw).numpy()
        c0 = int(inp.D_offsets[t])
        np.testing.assert_allclose(out[:, c0:c0 + D], ref, rtol=1e-6, atol=1e-6)


def test_forward_nobag_against_torch_embedding(lib=None):
    s = synth.Spec("nb", 1, (9,), (8,), 0, ("fixed", 1), ("uniform",), "none", False,
                   "f32", "dense", nobag_tokens=40, seed=77)
    inp = synth.generate(s)
    W = _weights(inp, 5)
    out = oracle.forward(_problem(inp), W, lib=lib)
    ref = torch.nn.functional.embedding(torch.from_numpy(inp.indices),
                                        torch.from_numpy(W.reshape(9, 8))).numpy()
    np.testing.assert_array_equal(out, ref)


def test_forward_nobag_multi_table_with_offsets(lib=None):
    """Nobag with offsets: lookup i of table t gets row W_t[indices[i]]."""
    s = synth.Spec("nb2", 2, (5, 6), (4, 4), 3, ("uniform", 0, 4), ("uniform",), "none", False,
                   "f32", "dense", seed=13)
    inp = synth.generate(s)
    W = _weights(inp, 9)
    out = oracle.forward(_problem(inp), W, lib=lib)
    for t in range(2):
        s0, s1 = int(inp.offsets[t * inp.B]), int(inp.offsets[(t + 1) * inp.B])
        w0 = int(inp.weights_offsets[t])
        for i in range(s0, s1):
            r = w0 + int(inp.indices[i]) * 4
            np.testing.assert_array_equal(out[i], W[r:r + 4])


@pytest.mark.parametrize("pooling,weighted", [("sum", True), ("mean", True), ("mean", False)])
def test_forward_is_adjoint_of_backward(pooling, weighted, lib=None):
    """<forward(W), G> == <W, dense backward(G)> for random W and G: ties the
    forward's coefficients, table offsets and columns to the backward's."""
    inp = _small(21, T=3, E=(6, 9, 4), D=(8, 4, 12), B=7, lens=("uniform", 0, 6),
                 pooling=pooling, weighted=weighted)
    W = _weights(inp, 3)
    out = oracle.forward(_problem(inp), W, lib=lib).astype(np.float64)
    Gb = inp.grad_output.astype(np.float64)
    lhs = float(np.sum(out * Gb))
    rows = np.arange(inp.total_rows)
    Gw, _ = oracle.row_grads(_problem(inp, grad=True), rows, lib=lib)
    rhs = 0.0
    for t in range(inp.T):
        r0, r1 = int(inp.hash_size_cumsum[t]), int(inp.hash_size_cumsum[t + 1])
        D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
        w0 = int(inp.weights_offsets[t])
        Wt = W[w0:w0 + (r1 - r0) * D].astype(np.float64).reshape(r1 - r0, D)
        rhs += float(np.sum(Wt * Gw[r0:r1, :D]))
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + abs(rhs)) + 1e-6, (lhs, rhs)


def test_forward_empty_bags_and_errors(lib=None):
    g, p, W = _golden()
    out = oracle.forward(p, W, lib=lib)
    assert np.all(out[0, 4:8] == 0)  # (t1, b0) is empty
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(replace(p, indices=np.array([0, 3, 1, 1, 0, 1])), W, lib=lib)
    assert e.value.status == "INDEX_OUT_OF_RANGE"
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(replace(p, offsets=np.array([0, 3, 2, 3, 6])), W, lib=lib)
    assert e.value.status == "BAD_OFFSETS"


_PINS = [test_forward_hand_golden,
         lambda lib: test_forward_against_torch_embedding_bag("sum", True, 1, lib),
         lambda lib: test_forward_against_torch_embedding_bag("mean", False, 2, lib),
         test_forward_nobag_against_torch_embedding, test_forward_nobag_multi_table_with_offsets,
         lambda lib: test_forward_is_adjoint_of_backward("mean", True, lib),
         test_forward_empty_bags_and_errors]

_MUTANTS = [
    ("forward mean scale dropped",
     r"const double scale = \(p->pooling == ORC_POOL_MEAN && L > 0\) \? 1\.0 / \(double\)L : 1\.0;",
     "const double scale = 1.0;"),
    ("forward weight dropped",
     r"scale \* \(p->per_sample_weights \? \(double\)p->per_sample_weights\[i\] : 1\.0\)", "scale"),
    ("forward column offset dropped",
     r"out\[\(int64_t\)b \* width \+ p->D_offsets\[t\] \+ d\]", "out[(int64_t)b * width + d]"),
    ("forward table base dropped", r"const float\* wr = W \+ woff \+", "const float* wr = W +"),
    ("forward nobag row of the bag", r"out\[i \* width \+ d\] = wr\[d\]", "out[(i - s) * width + d] = wr[d]"),
]


def _mutant_lib(tmp, desc, pattern, repl):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "sgb_oracle.c")).read()
    new, n = re.subn(pattern, repl, src)
    assert n >= 1, f"mutant '{desc}' did not apply"
    path = os.path.join(tmp, "m.c")
    with open(path, "w") as f:
        f.write(new)
    out = os.path.join(tmp, f"lib_{abs(hash(desc))}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", path, "-o", out, "-lm"])
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("desc,pattern,repl", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_forward_planted_mistakes(desc, pattern, repl):
    """Every planted forward mistake in a copy of the oracle fails at least one pin."""
    with tempfile.TemporaryDirectory() as tmp:
        lib = _mutant_lib(tmp, desc, pattern, repl)
        caught = 0
        for pin in _PINS:
            try:
                pin(lib=lib)
            except Exception:
                caught += 1
        assert caught > 0, f"no pin catches: {desc}"
