"""GPU parity of fp16 (IEEE binary16) weight rows under SGD and row-wise
Adagrad, rounded to nearest even or stochastically, against the oracle.

Both sides round their own fp32 result with the same rule and, for
stochastic rounding, the same Philox word; those fp32 results agree to the
fp32 tolerance but can straddle an fp16 rounding boundary (the kernels' fp32
coefficients and pair sums), so an element may differ by one fp16 spacing:
each element must lie within two spacings plus the fp32 tolerance of the
oracle's, and at most 1 in 10^3 elements may differ.  Untouched rows and
momentum are checked as for fp32 rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, oracle_problem, row_elements, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sgb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_gradient_backward_amd as m
    return m


_initial: dict = {}


def initial_f16(inp, mode):
    """Initial fp16 weights (IEEE nearest even of the seeded fp32 draw) and
    momentum, drawn once per input set (the draws advance their generators)."""
    key = (id(inp), mode)
    if key not in _initial:
        w0 = synth.initial_weights(inp).astype(np.float16)
        mom0 = synth.initial_momentum(inp) if mode == "rowwise_adagrad" else None
        _initial[key] = (inp, w0, mom0)
    return _initial[key][1], _initial[key][2]


def run_f16(sgb, inp, mode, thr, stochastic, seed, offset, lr=0.02, eps=1e-6):
    dev = to_dev(inp)
    w0, mom0 = initial_f16(inp, mode)
    w = torch.from_numpy(w0.copy()).cuda()
    mom = None if mom0 is None else torch.from_numpy(mom0).cuda()
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, thr)
    B = inp.B if inp.offsets is not None else 0
    ws = plan.workspace(inp.N, B)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode, weights=w,
                  momentum=mom, lr=lr, eps=eps, workspace=ws, stochastic_rounding=stochastic,
                  sr_seed=seed, sr_offset=offset)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"
    return (w0.view(np.uint16), w.cpu().numpy().view(np.uint16), mom0,
            None if mom is None else mom.cpu().numpy())


def check_f16(sgb, inp, mode, thr, stochastic, seed=20261203, offset=11, lr=0.02, eps=1e-6):
    w0h, wh, mom0, gm = run_f16(sgb, inp, mode, thr, stochastic, seed, offset, lr, eps)
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    touched = np.unique(keys)
    elems, valid, D = row_elements(inp, touched)
    G, _ = oracle.row_grads(oracle_problem(inp), touched)
    rows0 = np.where(valid, w0h[elems], 0).astype(np.uint16)
    rows, emom = oracle.update_rows_f16(mode, G, D, rows0,
                                        None if mom0 is None else mom0[touched], touched,
                                        lr=lr, eps=eps, stochastic=stochastic, seed=seed,
                                        offset=offset)
    got = wh[elems]
    diff = (got != rows) & valid
    n = int(valid.sum())
    if diff.any():
        g = got[diff].view(np.float16).astype(np.float64)
        e = rows[diff].view(np.float16).astype(np.float64)
        mag = np.maximum(np.abs(g), np.abs(e))
        spacing = np.where(mag < 2.0 ** -14, 2.0 ** -24,
                           np.ldexp(1.0, np.frexp(np.maximum(mag, 2.0 ** -14))[1] - 11))
        bound = 2 * spacing + 1e-4 + 1e-5 * np.abs(e)
        assert np.all(np.abs(g - e) <= bound), "fp16 rows differ beyond two roundings"
        assert diff.sum() <= max(2, n // 1000), f"{int(diff.sum())} of {n} fp16 elements differ"
    mask = np.ones(wh.shape[0], bool)
    mask[elems[valid]] = False
    assert np.array_equal(wh[mask], w0h[mask]), "untouched rows changed"
    if mode == "rowwise_adagrad":
        assert_close(gm[touched], emom, None, "momentum")
        mm = np.ones(gm.shape[0], bool)
        mm[touched] = False
        assert np.array_equal(gm[mm].view(np.uint32), mom0[mm].view(np.uint32))
    return wh


@pytest.mark.parametrize("stochastic", [True, False])
@pytest.mark.parametrize("mode", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("thr", [8, 2**31 - 1])
def test_f16_bags(sgb, mode, stochastic, thr):
    """Mixed widths (narrow, 256-column blocks, 1024 and 2048-wide rows),
    Zipf ids with runs both sides of the threshold, mean pooling with
    weights."""
    s = synth.Spec("f16_bags", 4, (700, 500, 300, 200), (16, 132, 1024, 2048), 129,
                   ("uniform", 0, 30), ("zipf", 1.2), "mean", True, "f32", mode, seed=47)
    check_f16(sgb, synth.generate(s), mode, thr, stochastic)


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_f16_nobag_sgd(sgb, grad_dtype):
    s = synth.Spec("f16_nobag", 1, (3000,), (768,), 0, ("fixed", 1), ("zipf", 1.1), "none",
                   False, grad_dtype, "sgd", nobag_tokens=2500, seed=53)
    check_f16(sgb, synth.generate(s), "sgd", 64, True)


def test_f16_long_runs_adagrad(sgb):
    """Hot rows over many chunks (ordered combine and its epilogue)."""
    s = synth.Spec("f16_hot", 2, (400, 600), (128, 48), 2000, ("uniform", 1, 12),
                   ("zipf", 2.0), "sum", True, "f32", "rowwise_adagrad", seed=59)
    check_f16(sgb, synth.generate(s), "rowwise_adagrad", 16, True)


def test_f16_small_values_and_draws(sgb):
    """Weights near the fp16 subnormal range (scaled down) and large steps
    (stochastic rounding through the subnormal grid); the same call twice is
    bit-identical and another offset draws other bits."""
    s = synth.Spec("f16_small", 2, (500, 800), (64, 128), 300, ("uniform", 1, 20),
                   ("zipf", 1.1), "sum", False, "f32", "sgd", weights_std=1e-5, seed=61)
    inp = synth.generate(s)
    a = check_f16(sgb, inp, "sgd", 32, True, seed=5, offset=1, lr=1e-4)
    b = check_f16(sgb, inp, "sgd", 32, True, seed=5, offset=1, lr=1e-4)
    c = check_f16(sgb, inp, "sgd", 32, True, seed=5, offset=2, lr=1e-4)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_f16_dense_unsupported(sgb):
    plan = sgb.Plan(np.array([0, 10]), np.array([0, 8]), "sum", 4)
    g = torch.zeros(1, 8, device="cuda")
    idx = torch.zeros(1, dtype=torch.int64, device="cuda")
    off = torch.tensor([0, 1], dtype=torch.int64, device="cuda")
    ws = plan.workspace(1, 1)
    with pytest.raises(sgb.SgbError, match="UNSUPPORTED"):
        plan.backward(g, idx, off, 1, None, "dense", grad=torch.zeros(80, device="cuda"),
                      weights=torch.zeros(80, dtype=torch.float16, device="cuda"), workspace=ws)
