"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped
coefficient, a wrong table offset, a transposed index, an unstable sort, a
wrong optimizer term) fails at least one of them; ``test_planted_mistakes``
checks exactly that by compiling mutated copies of the oracle source.
"""
import itertools
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


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _golden_two_tables():
    g = _load("hand_two_tables_mean_weighted.json")
    p = oracle.Problem(T=g["T"], B=g["B"], hash_size_cumsum=np.array(g["hash_size_cumsum"]),
                       D_offsets=np.array(g["D_offsets"]), offsets=np.array(g["offsets"]),
                       indices=np.array(g["indices"]),
                       per_sample_weights=np.array(g["per_sample_weights"], np.float32),
                       pooling=g["pooling"], grad_output=np.array(g["grad_output"], np.float32))
    return g, p


def _golden_nobag():
    g = _load("hand_nobag_bf16.json")
    p = oracle.Problem(T=1, B=0, hash_size_cumsum=np.array([0, g["E"]]),
                       D_offsets=np.array([0, g["D"]]), offsets=None,
                       indices=np.array(g["indices"]), per_sample_weights=None, pooling="none",
                       grad_output=synth.bf16_bits(np.array(g["grad_output"], np.float32)))
    return g, p


def _problem(inp: synth.Inputs) -> oracle.Problem:
    return oracle.Problem(T=inp.T, B=inp.B, hash_size_cumsum=inp.hash_size_cumsum,
                          D_offsets=inp.D_offsets, offsets=inp.offsets, indices=inp.indices,
                          per_sample_weights=inp.per_sample_weights, pooling=inp.spec.pooling,
                          grad_output=inp.grad_output)


# ---------------------------------------------------------------- hand-worked

def test_hand_two_tables_linearize_and_runs(lib=None):
    g, p = _golden_two_tables()
    keys, infos, coefs = oracle.linearize(p, lib=lib)
    assert keys.tolist() == g["expected_keys"]
    assert infos.tolist() == g["expected_infos"]
    assert coefs.tolist() == g["expected_coefs"]
    for thr, longs in g["expected_long_run_ids"].items():
        r = oracle.runs(keys, infos, int(thr), lib=lib)
        assert r["sorted_keys"].tolist() == g["expected_sorted_keys"]
        assert r["sorted_infos"].tolist() == g["expected_sorted_infos"]
        assert r["sorted_pos"].tolist() == g["expected_sorted_pos"]
        assert r["unique_ids"].tolist() == g["expected_unique_ids"]
        assert r["run_lengths"].tolist() == g["expected_run_lengths"]
        assert r["cumulative"].tolist() == g["expected_cumulative"]
        assert r["long_run_ids"].tolist() == longs


def test_hand_two_tables_grads_and_updates(lib=None):
    g, p = _golden_two_tables()
    G, hits = oracle.row_grads(p, np.array(g["expected_rows"]), lib=lib)
    assert G.tolist() == g["expected_G"]
    assert hits.tolist() == g["expected_hits"]
    s = g["sgd"]
    w, _ = oracle.update_rows("sgd", G[[s["row"]]][:, :4], np.array([4]),
                              np.array([s["w0"]], np.float32), None, lr=s["lr"], lib=lib)
    assert w[0].tolist() == s["expected"]
    a = g["adagrad"]
    w, m = oracle.update_rows("rowwise_adagrad", G[[a["row"]]], np.array([8]),
                              np.array([a["w0"]], np.float32), np.array([a["m0"]], np.float32),
                              lr=a["lr"], eps=a["eps"], lib=lib)
    assert w[0].tolist() == a["expected_w"]
    assert m[0] == a["expected_m"]
    d = g["dense_accumulate"]
    w, _ = oracle.update_rows("dense", G[[d["row"]]], np.array([8]),
                              np.array([d["out0"]], np.float32), None, accumulate=True, lib=lib)
    assert w[0].tolist() == d["expected"]
    w, _ = oracle.update_rows("dense", G[[d["row"]]], np.array([8]),
                              np.array([d["out0"]], np.float32), None, accumulate=False, lib=lib)
    assert w[0].tolist() == g["expected_G"][d["row"]]


def test_hand_nobag_bf16(lib=None):
    g, p = _golden_nobag()
    keys, infos, coefs = oracle.linearize(p, lib=lib)
    assert keys.tolist() == g["expected_keys"]
    assert infos.tolist() == g["expected_infos"]
    assert coefs.tolist() == [1.0] * 4
    r = oracle.runs(keys, infos, 2, lib=lib)
    assert r["sorted_keys"].tolist() == g["expected_sorted_keys"]
    assert r["sorted_infos"].tolist() == g["expected_sorted_infos"]
    assert r["unique_ids"].tolist() == g["expected_unique_ids"]
    assert r["run_lengths"].tolist() == g["expected_run_lengths"]
    assert r["cumulative"].tolist() == g["expected_cumulative"]
    assert r["long_run_ids"].tolist() == [1]
    G, hits = oracle.row_grads(p, np.array(g["expected_rows"]), lib=lib)
    assert G.tolist() == g["expected_G"]
    assert hits.tolist() == [1, 0, 3]


# ---------------------------------------------------------------- small random problems

def _small(seed, T=3, E=(7, 5, 11), D=(4, 12, 8), B=6, lens=("uniform", 0, 5), pooling="sum",
           weighted=False, grad_dtype="f32", zipf=None):
    s = synth.Spec("small", T, tuple(E), tuple(D), B, lens,
                   ("zipf", zipf) if zipf else ("uniform",), pooling, weighted, grad_dtype,
                   "dense", seed=seed)
    return synth.generate(s)


def _grad_f64(inp):
    g = inp.grad_output
    if g.dtype == np.uint16:
        g = synth.bf16_to_f32(g)
    return g.astype(np.float64)


def _torch_embedding_bag_grads(inp):
    """Row gradients from torch's own embedding_bag / embedding autograd (fp64, CPU)."""
    out = []
    g = torch.from_numpy(_grad_f64(inp))
    for t in range(inp.T):
        E = int(inp.hash_size_cumsum[t + 1] - inp.hash_size_cumsum[t])
        D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
        w = torch.zeros(E, D, dtype=torch.float64, requires_grad=True)
        if inp.spec.pooling == "none":
            s, e = (0, inp.N) if inp.offsets is None else (int(inp.offsets[t * inp.B]),
                                                            int(inp.offsets[(t + 1) * inp.B]))
            y = torch.nn.functional.embedding(torch.from_numpy(inp.indices[s:e]), w)
            y.backward(g[s:e, :D])
        else:
            off = inp.offsets[t * inp.B:(t + 1) * inp.B + 1]
            idx = torch.from_numpy(inp.indices[off[0]:off[-1]])
            o = torch.from_numpy(off[:-1] - off[0])
            psw = None
            if inp.per_sample_weights is not None:
                psw = torch.from_numpy(inp.per_sample_weights[off[0]:off[-1]].astype(np.float64))
            y = torch.nn.functional.embedding_bag(idx, w, o, mode=inp.spec.pooling,
                                                  per_sample_weights=psw)
            y.backward(g[:, int(inp.D_offsets[t]):int(inp.D_offsets[t]) + D])
        out.append(w.grad.numpy())
    return out


def _oracle_all_rows(inp, lib=None):
    p = _problem(inp)
    rows = np.arange(inp.total_rows)
    G, hits = oracle.row_grads(p, rows, lib=lib)
    return G, hits


@pytest.mark.parametrize("pooling,weighted", [("sum", False), ("sum", True), ("mean", False)])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_against_torch_embedding_bag(pooling, weighted, seed, lib=None):
    inp = _small(seed, pooling=pooling, weighted=weighted)
    G, _ = _oracle_all_rows(inp, lib=lib)
    ref = _torch_embedding_bag_grads(inp)
    for t in range(inp.T):
        r0, r1 = inp.hash_size_cumsum[t], inp.hash_size_cumsum[t + 1]
        D = ref[t].shape[1]
        np.testing.assert_allclose(G[r0:r1, :D], ref[t], rtol=1e-12, atol=1e-12)
        assert np.all(G[r0:r1, D:] == 0)


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_nobag_against_torch_embedding(grad_dtype, lib=None):
    s = synth.Spec("nb", 1, (9,), (8,), 0, ("fixed", 1), ("uniform",), "none", False,
                   grad_dtype, "dense", nobag_tokens=40, seed=77)
    inp = synth.generate(s)
    G, _ = _oracle_all_rows(inp, lib=lib)
    ref = _torch_embedding_bag_grads(inp)
    np.testing.assert_allclose(G, ref[0], rtol=1e-12, atol=1e-12)


def test_nobag_multi_table_with_offsets(lib=None):
    """Nobag with T=2 tables and offsets: lookup i of table t reads grad_output[i]."""
    s = synth.Spec("nb2", 2, (5, 6), (4, 4), 3, ("uniform", 0, 4), ("uniform",), "none", False,
                   "f32", "dense", seed=78)
    inp = synth.generate(s, with_grad=False)
    inp.grad_output = inp.rngs["grad_output"].standard_normal((inp.N, 4), dtype=np.float32)
    G, _ = _oracle_all_rows(inp, lib=lib)
    ref = _torch_embedding_bag_grads(inp)
    np.testing.assert_allclose(G[:5], ref[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(G[5:], ref[1], rtol=1e-12, atol=1e-12)
    keys, infos, _ = oracle.linearize(_problem(inp), lib=lib)
    assert np.array_equal(infos // 2, np.arange(inp.N))
    assert np.array_equal(infos % 2, (np.arange(inp.N) >= inp.offsets[3]).astype(np.int64))


@pytest.mark.parametrize("seed", [4, 5])
def test_one_hot_matmul_mean_weighted(seed, lib=None):
    """G_t = A_t^T @ grad_t with A_t[b, r] = sum of weight/L over lookups of bag b on row r."""
    inp = _small(seed, pooling="mean", weighted=True, grad_dtype="bf16")
    G, _ = _oracle_all_rows(inp, lib=lib)
    g = _grad_f64(inp)
    for t in range(inp.T):
        E = int(inp.hash_size_cumsum[t + 1] - inp.hash_size_cumsum[t])
        D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
        A = np.zeros((inp.B, E))
        for b in range(inp.B):
            s, e = inp.offsets[t * inp.B + b], inp.offsets[t * inp.B + b + 1]
            for i in range(s, e):
                A[b, inp.indices[i]] += float(inp.per_sample_weights[i]) / (e - s)
        ref = A.T @ g[:, int(inp.D_offsets[t]):int(inp.D_offsets[t]) + D]
        r0 = inp.hash_size_cumsum[t]
        np.testing.assert_allclose(G[r0:r0 + E, :D], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pooling,weighted", [("sum", True), ("mean", True), ("mean", False)])
def test_mass_invariant(pooling, weighted, lib=None):
    """Per table and column: sum over rows of G equals the pooled mass of grad_output."""
    inp = _small(9, pooling=pooling, weighted=weighted, zipf=1.3, B=40)
    G, _ = _oracle_all_rows(inp, lib=lib)
    g = _grad_f64(inp)
    for t in range(inp.T):
        D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
        mass = np.zeros(D)
        for b in range(inp.B):
            s, e = inp.offsets[t * inp.B + b], inp.offsets[t * inp.B + b + 1]
            w = inp.per_sample_weights[s:e].astype(np.float64) if weighted else np.ones(e - s)
            c = w.sum() / (e - s) if (pooling == "mean" and e > s) else w.sum()
            mass += c * g[b, int(inp.D_offsets[t]):int(inp.D_offsets[t]) + D]
        r0, r1 = inp.hash_size_cumsum[t], inp.hash_size_cumsum[t + 1]
        np.testing.assert_allclose(G[r0:r1, :D].sum(axis=0), mass, rtol=1e-11, atol=1e-11)


def test_special_permutation_and_column_sums(lib=None):
    # all-distinct length-1 bags: G is a permutation of grad_output rows
    B, E, D = 16, 16, 8
    perm = np.random.default_rng(3).permutation(E)
    g = np.random.default_rng(4).standard_normal((B, D)).astype(np.float32)
    p = oracle.Problem(1, B, np.array([0, E]), np.array([0, D]), np.arange(B + 1), perm, None,
                       "sum", g)
    G, hits = oracle.row_grads(p, np.arange(E), lib=lib)
    assert np.array_equal(G[perm], g.astype(np.float64))
    assert np.all(hits == 1)
    # every lookup on one row: G is the column sum of the pooled gradient
    lens = np.array([3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8, 9, 7, 9, 3])
    off = np.concatenate([[0], np.cumsum(lens)])
    p = oracle.Problem(1, B, np.array([0, E]), np.array([0, D]), off,
                       np.full(off[-1], 5), None, "sum", g)
    G, hits = oracle.row_grads(p, np.array([5]), lib=lib)
    np.testing.assert_allclose(G[0], (lens[:, None] * g.astype(np.float64)).sum(0), rtol=1e-13)
    assert hits[0] == off[-1]
    # mean with constant L = k equals sum / k
    k = 4
    idx = np.random.default_rng(5).integers(0, E, B * k)
    p_sum = oracle.Problem(1, B, np.array([0, E]), np.array([0, D]), np.arange(B + 1) * k, idx,
                           None, "sum", g)
    p_mean = oracle.Problem(1, B, np.array([0, E]), np.array([0, D]), np.arange(B + 1) * k, idx,
                            None, "mean", g)
    Gs, _ = oracle.row_grads(p_sum, np.arange(E), lib=lib)
    Gm, _ = oracle.row_grads(p_mean, np.arange(E), lib=lib)
    np.testing.assert_allclose(Gm, Gs / k, rtol=1e-14)


# ---------------------------------------------------------------- run structure

@pytest.mark.parametrize("seed", range(6))
def test_runs_brute_force(seed, lib=None):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 60))
    keys = rng.integers(0, 9, n)
    infos = rng.integers(0, 1000, n)
    thr = int(rng.integers(1, 6))
    r = oracle.runs(keys, infos, thr, lib=lib)
    order = sorted(range(n), key=lambda i: keys[i])  # Python's sort is stable
    assert r["sorted_pos"].tolist() == order
    assert r["sorted_keys"].tolist() == [int(keys[i]) for i in order]
    assert r["sorted_infos"].tolist() == [int(infos[i]) for i in order]
    groups = [(k, len(list(grp))) for k, grp in itertools.groupby(keys[order].tolist())]
    u, c = np.unique(keys, return_counts=True)
    assert r["unique_ids"].tolist() == [k for k, _ in groups] == u.tolist()
    assert r["run_lengths"].tolist() == [m for _, m in groups] == c.tolist()
    assert r["cumulative"].tolist() == [0] + np.cumsum(c).tolist()
    assert r["long_run_ids"].tolist() == [i for i, (_, m) in enumerate(groups) if m >= thr]
    assert r["num_runs"] == len(groups)


def test_runs_invariants_on_generated(lib=None):
    inp = _small(11, T=4, E=(50, 3, 70, 9), D=(4, 4, 8, 16), B=30, zipf=1.1, lens=("poisson", 5))
    keys, infos, _ = oracle.linearize(_problem(inp), lib=lib)
    r = oracle.runs(keys, infos, 7, lib=lib)
    assert r["run_lengths"].sum() == inp.N and r["cumulative"][-1] == inp.N
    assert np.all(np.diff(r["unique_ids"]) > 0)
    hsc = inp.hash_size_cumsum
    for k in range(r["num_runs"]):
        a, b = r["cumulative"][k], r["cumulative"][k + 1]
        t = r["sorted_infos"][a:b] // inp.B
        assert np.all(hsc[t] <= r["unique_ids"][k]) and np.all(r["unique_ids"][k] < hsc[t + 1])
        assert np.all(np.diff(r["sorted_infos"][a:b]) >= 0)  # stable => infos non-decreasing
    longs = set(r["long_run_ids"].tolist())
    assert longs == {k for k in range(r["num_runs"]) if r["run_lengths"][k] >= 7}


# ---------------------------------------------------------------- optimizers

def test_sgd_fused_equals_dense_then_step(lib=None):
    inp = _small(12, pooling="mean", weighted=True)
    G, _ = _oracle_all_rows(inp, lib=lib)
    D = np.repeat(np.diff(inp.D_offsets), np.diff(inp.hash_size_cumsum)).astype(np.int32)
    w0 = np.random.default_rng(1).standard_normal(G.shape).astype(np.float32)
    w, _ = oracle.update_rows("sgd", G, D, w0, None, lr=0.25, lib=lib)
    dense, _ = oracle.update_rows("dense", G, D, None, None, lib=lib)
    for k in range(G.shape[0]):
        np.testing.assert_allclose(w[k, :D[k]], w0[k, :D[k]] - 0.25 * G[k, :D[k]], rtol=1e-6,
                                   atol=1e-6)
        np.testing.assert_allclose(dense[k, :D[k]], G[k, :D[k]], rtol=1e-7, atol=1e-30)


def test_adagrad_single_occurrence_closed_form(lib=None):
    g = np.array([[0.5, -1.5, 2.0, 0.25, 3.0, -0.75, 1.0, 0.0]])
    w0 = np.array([[1.0, 2.0, -1.0, 0.5, 0.0, 0.0, 3.0, -2.0]], np.float32)
    lr, eps = 0.01, 1e-8
    w, m = oracle.update_rows("rowwise_adagrad", g, np.array([8]), w0, np.zeros(1, np.float32),
                              lr=lr, eps=eps, lib=lib)
    rms = np.sqrt(np.mean(g ** 2))
    np.testing.assert_allclose(w, w0 - np.float32(lr) * g / (rms + np.float32(eps)), rtol=1e-7)
    np.testing.assert_allclose(m, [np.mean(g ** 2)], rtol=1e-7)
    # a second step with the grown state uses sqrt(m0 + mean(G^2))
    w2, m2 = oracle.update_rows("rowwise_adagrad", g, np.array([8]), w, m, lr=lr, eps=eps, lib=lib)
    np.testing.assert_allclose(m2, 2 * m, rtol=1e-7)
    np.testing.assert_allclose(w2, w - np.float32(lr) * g / (np.sqrt(2) * rms + eps), rtol=1e-6)
    # eps sits outside the square root: G = [3, 4, 0, 0], mean square 6.25, sqrt 2.5,
    # + eps 0.5 = 3, lr 3 -> multiplier exactly 1
    w3, m3 = oracle.update_rows("rowwise_adagrad", np.array([[3.0, 4.0, 0.0, 0.0]]),
                                np.array([4]), np.zeros((1, 4), np.float32),
                                np.zeros(1, np.float32), lr=3.0, eps=0.5, lib=lib)
    assert w3[0].tolist() == [-3.0, -4.0, 0.0, 0.0] and m3[0] == 6.25


def test_untouched_rows_have_no_hits(lib=None):
    inp = _small(13, B=3, lens=("uniform", 0, 2))
    G, hits = _oracle_all_rows(inp, lib=lib)
    keys, _, _ = oracle.linearize(_problem(inp), lib=lib)
    touched = set(keys.tolist())
    for r in range(inp.total_rows):
        assert (hits[r] > 0) == (r in touched)
        if r not in touched:
            assert np.all(G[r] == 0)


# ---------------------------------------------------------------- validation

def test_validation_errors(lib=None):
    _, p = _golden_two_tables()
    assert oracle.validate(p, lib=lib) == "OK"
    bad = dict(offsets=np.array([0, 2, 1, 3, 7]))
    assert oracle.validate(replace(p, **bad), lib=lib) == "BAD_OFFSETS"
    bad = dict(offsets=np.array([0, 2, 3, 3, 6]))
    assert oracle.validate(replace(p, **bad), lib=lib) == "BAD_OFFSETS"
    bad = dict(indices=np.array([2, 0, 3, 1, 1, 0, 1]))  # 3 >= E_0 = 3
    assert oracle.validate(replace(p, **bad), lib=lib) == \
        "INDEX_OUT_OF_RANGE"
    bad = dict(indices=np.array([2, 0, 2, 1, 1, -1, 1]))
    assert oracle.validate(replace(p, **bad), lib=lib) == \
        "INDEX_OUT_OF_RANGE"
    bad = dict(D_offsets=np.array([0, 4, 14]))  # D_1 = 10, not a multiple of 4
    assert oracle.validate(replace(p, **bad), lib=lib) == \
        "INVALID_ARGUMENT"
    bad = dict(hash_size_cumsum=np.array([0, 3, 3]))
    assert oracle.validate(replace(p, **bad), lib=lib) == \
        "INVALID_ARGUMENT"
    _, q = _golden_nobag()
    assert oracle.validate(q, lib=lib) == "OK"
    wq = replace(q, per_sample_weights=np.ones(4, np.float32))
    assert oracle.validate(wq, lib=lib) == "UNSUPPORTED"
    with pytest.raises(oracle.OracleError):
        oracle.row_grads(replace(p, offsets=np.array([0, 2, 1, 3, 7])),
                         np.arange(5), lib=lib)


# ---------------------------------------------------------------- planted mistakes

_PINS = [test_hand_two_tables_linearize_and_runs, test_hand_two_tables_grads_and_updates,
         test_hand_nobag_bf16, lambda lib: test_against_torch_embedding_bag("sum", True, 1, lib),
         lambda lib: test_against_torch_embedding_bag("mean", False, 2, lib),
         lambda lib: test_nobag_against_torch_embedding("bf16", lib),
         lambda lib: test_one_hot_matmul_mean_weighted(4, lib),
         lambda lib: test_runs_brute_force(3, lib), test_sgd_fused_equals_dense_then_step,
         test_adagrad_single_occurrence_closed_form, test_nobag_multi_table_with_offsets,
         test_validation_errors]

# (description, regex in sgb_oracle.c, replacement)
_MUTANTS = [
    ("mean scale dropped",
     r"\(p->pooling == ORC_POOL_MEAN && L > 0\) \? 1\.0 / \(double\)L\s*\n\s*: 1\.0;", "1.0;"),
    ("weight dropped in grads", r"\? \(double\)p->per_sample_weights\[i\]\n(\s*): 1\.0\);",
     "? 1.0\n\\1: 1.0);"),
    ("table offset dropped in key", r"keys\[i\] = p->hash_size_cumsum\[t\] \+ p->indices\[i\];",
     "keys[i] = p->indices[i];"),
    ("wrong column offset", r"orc_grad\(p, b, width, p->D_offsets\[t\] \+ d\)",
     "orc_grad(p, b, width, d)"),
    ("unstable tie order", r"if \(x->pos != y->pos\) return x->pos < y->pos \? -1 : 1;",
     "if (x->pos != y->pos) return x->pos < y->pos ? 1 : -1;"),
    ("long test uses >", r"if \(run_lengths\[r\] >= thr\)", "if (run_lengths[r] > thr)"),
    ("sgd sign", r"\(double\)w\[d\] - \(double\)lr \* g\[d\]", "(double)w[d] + (double)lr * g[d]"),
    ("adagrad eps inside sqrt", r"sqrt\(m\) \+ \(double\)eps", "sqrt(m + (double)eps)"),
    ("adagrad old state", r"double mult = \(double\)lr / \(sqrt\(m\)",
     "double mult = (double)lr / (sqrt((double)mom[k])"),
    ("adagrad sum not mean", r"sumsq / \(double\)Dk", "sumsq"),
    ("nobag info", r"infos\[i\] = nobag \? i \* \(int64_t\)p->T \+ t", "infos[i] = nobag ? i"),
    ("bf16 widened wrong", r"\(\(uint32_t\)h\) << 16", "((uint32_t)h) << 15"),
    ("accumulate ignored", r"w\[d\] = accumulate \? \(float\)\(\(double\)w\[d\] \+ g\[d\]\) : \(float\)g\[d\];",
     "w[d] = (float)g[d];"),
    ("offset check missing", r"if \(p->offsets\[k \+ 1\] < p->offsets\[k\]\) return ORC_BAD_OFFSETS;",
     "(void)0;"),
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
def test_planted_mistakes(desc, pattern, repl):
    """Every planted mistake in a copy of the oracle fails at least one pin."""
    with tempfile.TemporaryDirectory() as tmp:
        lib = _mutant_lib(tmp, desc, pattern, repl)
        caught = 0
        for pin in _PINS:
            try:
                pin(lib=lib)
            except Exception:
                caught += 1
        assert caught > 0, f"no pin catches: {desc}"
