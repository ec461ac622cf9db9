"""GPU parity of INT8 row-wise quantized weight rows (SGD and row-wise
Adagrad) against the oracle.

A row is D uint8 codes followed by its fp32 scale and bias; after the update
both sides requantize their own fp32 row with the same rule.  Those fp32 rows
agree to the fp32 tolerance, not always to the bit (the kernels' fp32
coefficient and fp32 pair sums), so a code sitting on a rounding boundary may
differ by one and the parameters by a few ulps.  Each row's scale and bias
must be within 1e-6 + 1e-5 |oracle|, each code within one of the oracle's, at
most 1 in 10^3 codes may differ, untouched bytes must be unchanged, and
momentum meets the usual tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, oracle_problem, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sgb():
    import sparse_gradient_backward_amd as m
    return m


def int8_layout(inp):
    E = np.diff(inp.hash_size_cumsum).astype(np.int64)
    D = np.diff(inp.D_offsets).astype(np.int64)
    woff8 = np.concatenate([[0], np.cumsum(E * (D + 8))]).astype(np.int64)
    return E, D, woff8


_initial: dict = {}


def initial_int8(inp, mode):
    """Initial INT8 rows (the oracle's quantization of the seeded fp32 draw)
    and momentum, drawn once per input set."""
    key = (id(inp), mode)
    if key not in _initial:
        E, D, woff8 = int8_layout(inp)
        w = synth.initial_weights(inp)
        buf = np.zeros(int(woff8[-1]), np.uint8)
        for t in range(inp.T):
            wt = w[inp.weights_offsets[t]:inp.weights_offsets[t + 1]].reshape(E[t], D[t])
            buf[woff8[t]:woff8[t + 1]] = oracle.i8_quantize(wt).ravel()
        mom0 = synth.initial_momentum(inp) if mode == "rowwise_adagrad" else None
        _initial[key] = (inp, buf, mom0)
    return _initial[key][1], _initial[key][2]


def check_int8(sgb, inp, mode, thr, lr=0.02, eps=1e-6):
    buf0, mom0 = initial_int8(inp, mode)
    dev = to_dev(inp)
    w = torch.from_numpy(buf0.copy()).cuda()
    mom = None if mom0 is None else torch.from_numpy(mom0).cuda()
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, thr)
    B = inp.B if inp.offsets is not None else 0
    ws = plan.workspace(inp.N, B)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode, weights=w,
                  momentum=mom, lr=lr, eps=eps, workspace=ws)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"
    got = w.cpu().numpy()
    E, D, woff8 = int8_layout(inp)
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    touched = np.unique(keys)
    t = np.searchsorted(inp.hash_size_cumsum, touched, side="right") - 1
    Dr = D[t]
    start = woff8[t] + (touched - inp.hash_size_cumsum[t]) * (Dr + 8)
    ldr = int(D.max()) + 8
    cols = np.arange(ldr)[None, :]
    valid = cols < (Dr + 8)[:, None]
    idx = np.where(valid, start[:, None] + cols, 0)
    G, _ = oracle.row_grads(oracle_problem(inp), touched)
    exp, emom = oracle.update_rows_int8(mode, G, Dr, np.where(valid, buf0[idx], 0), None if mom0 is None
                                        else mom0[touched], lr=lr, eps=eps)
    gr = np.where(valid, got[idx], 0).astype(np.uint8)
    ncode = 0
    bad = 0
    for k in range(len(touched)):
        d = int(Dr[k])
        gq = gr[k, d:d + 8].copy().view(np.float32)
        eq = exp[k, d:d + 8].copy().view(np.float32)
        assert np.all(np.abs(gq - eq) <= 1e-6 + 1e-5 * np.abs(eq)), \
            f"row {touched[k]}: scale/bias gpu {gq} oracle {eq}"
        dc = np.abs(gr[k, :d].astype(int) - exp[k, :d].astype(int))
        assert dc.max() <= 1, f"row {touched[k]}: a code differs by {dc.max()}"
        bad += int((dc > 0).sum())
        ncode += d
    assert bad <= max(2, ncode // 1000), f"{bad} of {ncode} codes differ"
    mask = np.ones(got.shape[0], bool)
    mask[idx[valid]] = False
    assert np.array_equal(got[mask], buf0[mask]), "untouched bytes changed"
    if mode == "rowwise_adagrad":
        gm = mom.cpu().numpy()
        assert_close(gm[touched], emom, None, "momentum")


@pytest.mark.parametrize("mode", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("thr", [8, 2**31 - 1])
def test_int8_bags(sgb, mode, thr):
    """Mixed widths (narrow, 256-column blocks and 1024-wide rows), Zipf ids
    with runs both sides of the threshold, mean pooling with weights."""
    s = synth.Spec("int8_bags", 4, (700, 500, 300, 900), (16, 132, 1024, 64), 129,
                   ("uniform", 0, 30), ("zipf", 1.2), "mean", True, "f32", mode, seed=37)
    check_int8(sgb, synth.generate(s), mode, thr)


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_int8_nobag_sgd(sgb, grad_dtype):
    s = synth.Spec("int8_nobag", 1, (3000,), (768,), 0, ("fixed", 1), ("zipf", 1.1), "none",
                   False, grad_dtype, "sgd", nobag_tokens=2500, seed=41)
    check_int8(sgb, synth.generate(s), "sgd", 64)


def test_int8_long_runs_adagrad(sgb):
    """Hot rows over many chunks (ordered combine, then the whole-row
    requantization by the last wave) beside narrow rows."""
    s = synth.Spec("int8_hot", 2, (400, 600), (256, 48), 2000, ("uniform", 1, 12),
                   ("zipf", 2.0), "sum", True, "f32", "rowwise_adagrad", seed=43)
    check_int8(sgb, synth.generate(s), "rowwise_adagrad", 16)


def test_int8_rejected_cases(sgb):
    g = torch.zeros(1, 2048, device="cuda")
    idx = torch.zeros(1, dtype=torch.int64, device="cuda")
    off = torch.tensor([0, 1], dtype=torch.int64, device="cuda")
    plan = sgb.Plan(np.array([0, 10]), np.array([0, 8]), "sum", 4)
    ws = plan.workspace(1, 1)
    with pytest.raises(sgb.SgbError, match="UNSUPPORTED"):   # a dense gradient is fp32
        plan.backward(g[:, :8].contiguous(), idx, off, 1, None, "dense",
                      grad=torch.zeros(80, device="cuda"),
                      weights=torch.zeros(160, dtype=torch.uint8, device="cuda"), workspace=ws)
