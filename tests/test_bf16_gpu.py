"""GPU parity of bf16 weight rows (SGD and row-wise Adagrad, stochastic
rounding from Philox4x32-10 or round-to-nearest-even) against the oracle.

Both sides form an fp32 value and round it to bf16 with the same random
word.  The two fp32 values agree to the fp32 tolerance but not always to the
bit: the kernels fold the per-sample weight and 1/L into one fp32
coefficient, and the short-run reducer adds pairs of products in fp32.  When
the two values straddle a bf16 rounding boundary, the bf16 results differ by
one ulp.  So each element must satisfy
|gpu - oracle| <= 2 ulp_bf16 + 1e-4 + 1e-5 |oracle|
(two roundings of values within the fp32 tolerance), and at most 1 element in
10^3 may differ at all: a wrong random word, or nearest-even in place of
stochastic rounding, changes about half of them.  Momentum is compared to the
usual tolerance; untouched rows must be bit-unchanged."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, oracle_problem, row_elements, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sgb():
    import sparse_gradient_backward_amd as m
    return m


_initial: dict = {}


def initial_bf16(inp, mode):
    """Initial bf16 weights (nearest-even of the seeded fp32 draw) and momentum,
    drawn once per input set (the draws advance their generators)."""
    key = (id(inp), mode)
    if key not in _initial:
        w0 = torch.from_numpy(synth.initial_weights(inp)).to(torch.bfloat16)
        mom0 = synth.initial_momentum(inp) if mode == "rowwise_adagrad" else None
        _initial[key] = (inp, w0, mom0)
    return _initial[key][1], _initial[key][2]


def run_bf16(sgb, inp, mode, thr, stochastic, seed, offset, lr=0.02, eps=1e-6):
    dev = to_dev(inp)
    w0, mom0 = initial_bf16(inp, mode)
    w = w0.cuda()
    mom = None if mom0 is None else torch.from_numpy(mom0).cuda()
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, thr)
    B = inp.B if inp.offsets is not None else 0
    ws = plan.workspace(inp.N, B)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode, weights=w,
                  momentum=mom, lr=lr, eps=eps, workspace=ws, stochastic_rounding=stochastic,
                  sr_seed=seed, sr_offset=offset)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"
    w0b = w0.view(torch.int16).numpy().view(np.uint16)
    wb = w.cpu().view(torch.int16).numpy().view(np.uint16)
    return w0b, wb, mom0, None if mom is None else mom.cpu().numpy()


def expected_bf16(inp, mode, w0b, mom0, stochastic, seed, offset, lr=0.02, eps=1e-6):
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    touched = np.unique(keys)
    elems, valid, D = row_elements(inp, touched)
    G, _ = oracle.row_grads(oracle_problem(inp), touched)
    rows0 = np.where(valid, w0b[elems], 0).astype(np.uint16)
    rows, mom = oracle.update_rows_bf16(mode, G, D, rows0, None if mom0 is None else mom0[touched],
                                        touched, lr=lr, eps=eps, stochastic=stochastic, seed=seed,
                                        offset=offset)
    return touched, elems, valid, rows, mom


def _bf(h):
    return float((np.uint32(h) << np.uint32(16)).view(np.float32))


def _describe(inp, mode, touched, elems, valid, got, rows, w0b, mom0, seed, offset):
    """Prints each differing element: its row and column, both bf16 values,
    the oracle's fp32 value before rounding and the rounding word."""
    G, hits = oracle.row_grads(oracle_problem(inp), touched)
    D = np.diff(inp.D_offsets)[np.searchsorted(inp.hash_size_cumsum, touched, side="right") - 1]
    w32 = (np.where(valid, w0b[elems], 0).astype(np.uint32) << 16).view(np.float32)
    f32, _ = oracle.update_rows(mode, G, D, w32, None if mom0 is None else mom0[touched],
                                lr=0.02, eps=1e-6)
    for r, c in np.argwhere((got != rows) & valid)[:10]:
        word = oracle.philox4x32_10((c // 4, touched[r] & 0xFFFFFFFF, touched[r] >> 32, offset),
                                    (seed & 0xFFFFFFFF, seed >> 32))[c % 4]
        print(f"[bf16] row {touched[r]} (D={D[r]}, lookups={hits[r]}) col {c}: gpu {_bf(got[r, c])!r} "
              f"oracle {_bf(rows[r, c])!r} fp32 {f32[r, c]!r} "
              f"(bits {int(np.float32(f32[r, c]).view(np.uint32)):08x}, word {int(word):08x})",
              flush=True)


def check_bf16(sgb, inp, mode, thr, stochastic, seed=20261202, offset=7):
    w0b, wb, mom0, gm = run_bf16(sgb, inp, mode, thr, stochastic, seed, offset)
    touched, elems, valid, rows, emom = expected_bf16(inp, mode, w0b, mom0, stochastic, seed,
                                                      offset)
    got = wb[elems]
    diff = (got != rows) & valid
    n = int(valid.sum())
    if diff.any():
        _describe(inp, mode, touched, elems, valid, got, rows, w0b, mom0, seed, offset)
        g = (got[diff].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        e = (rows[diff].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(g), np.abs(e)))[1] - 8)
        bound = 2 * ulp + 1e-4 + 1e-5 * np.abs(e)
        assert np.all(np.abs(g - e) <= bound), "bf16 rows differ beyond two roundings"
        assert diff.sum() <= max(2, n // 1000), f"{int(diff.sum())} of {n} bf16 elements differ"
    mask = np.ones(wb.shape[0], bool)
    mask[elems[valid]] = False
    assert np.array_equal(wb[mask], w0b[mask]), "untouched rows changed"
    if mode == "rowwise_adagrad":
        assert_close(gm[touched], emom, None, "momentum")
        mm = np.ones(gm.shape[0], bool)
        mm[touched] = False
        assert np.array_equal(gm[mm].view(np.uint32), mom0[mm].view(np.uint32))
    return wb


@pytest.mark.parametrize("stochastic", [True, False])
@pytest.mark.parametrize("mode", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("thr", [8, 2**31 - 1])
def test_bf16_bags(sgb, mode, stochastic, thr):
    """Mixed widths (narrow, 256-column blocks and wider rows), Zipf ids with
    runs both sides of the threshold, mean pooling with weights."""
    s = synth.Spec("bf16_bags", 4, (700, 500, 300, 900), (16, 132, 1024, 64), 129,
                   ("uniform", 0, 30), ("zipf", 1.2), "mean", True, "f32", mode, seed=17)
    check_bf16(sgb, synth.generate(s), mode, thr, stochastic)


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_bf16_nobag_sgd(sgb, grad_dtype):
    s = synth.Spec("bf16_nobag", 1, (3000,), (768,), 0, ("fixed", 1), ("zipf", 1.1), "none",
                   False, grad_dtype, "sgd", nobag_tokens=2500, seed=23)
    check_bf16(sgb, synth.generate(s), "sgd", 64, True)


def test_bf16_long_runs_adagrad(sgb):
    """One hot row over many chunks (the long-run reducer's ordered combine
    and its epilogue), plus narrow rows."""
    s = synth.Spec("bf16_hot", 2, (400, 600), (128, 48), 2000, ("uniform", 1, 12),
                   ("zipf", 2.0), "sum", True, "f32", "rowwise_adagrad", seed=29)
    check_bf16(sgb, synth.generate(s), "rowwise_adagrad", 16, True)


def test_bf16_stochastic_rounding_draws(sgb):
    """Same call twice: bit-identical; another offset draws other bits; and
    the fraction of elements rounded up matches the fractions the fp32 values
    call for (the oracle's rows with nearest-even differ from stochastic ones
    on about half the non-exact elements)."""
    s = synth.Spec("bf16_draws", 2, (500, 800), (64, 128), 300, ("uniform", 1, 20),
                   ("zipf", 1.1), "sum", False, "f32", "sgd", seed=31)
    inp = synth.generate(s)
    a = check_bf16(sgb, inp, "sgd", 32, True, seed=5, offset=1)
    b = check_bf16(sgb, inp, "sgd", 32, True, seed=5, offset=1)
    c = check_bf16(sgb, inp, "sgd", 32, True, seed=5, offset=2)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_bf16_dense_unsupported(sgb):
    plan = sgb.Plan(np.array([0, 10]), np.array([0, 8]), "sum", 4)
    g = torch.zeros(1, 8, device="cuda")
    idx = torch.zeros(1, dtype=torch.int64, device="cuda")
    off = torch.tensor([0, 1], dtype=torch.int64, device="cuda")
    ws = plan.workspace(1, 1)
    # a bf16 weights buffer alongside a dense gradient: rejected by the library
    with pytest.raises(sgb.SgbError, match="UNSUPPORTED"):
        plan.backward(g, idx, off, 1, None, "dense", grad=torch.zeros(80, device="cuda"),
                      weights=torch.zeros(80, dtype=torch.bfloat16, device="cuda"), workspace=ws)
