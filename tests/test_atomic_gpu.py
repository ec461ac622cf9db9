"""GPU parity of the atomic scatter-add baseline (libsgb_atomic.so) against
the CPU oracle: dense gradient (fresh and accumulated) and SGD, bag and
nobag, fp32 and bf16 gradients.  Float atomics add in no fixed order, so the
comparison is to the tolerance; an integer-valued case with power-of-two
coefficients is exact in any order and compared bit for bit."""
import numpy as np
import pytest
import torch

import synth
from harness import assert_close, expected_rows, initial_buffers, oracle_problem, row_elements, \
    to_dev
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def atomic():
    import sparse_gradient_backward_amd.atomic as a
    return a


def run_atomic(atomic, inp, mode, accumulate, lr):
    tables = atomic.AtomicTables(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling)
    dev = to_dev(inp)
    out0, _ = initial_buffers(inp, mode, accumulate)
    out = torch.from_numpy(out0).cuda()
    scale = -lr if mode == "sgd" else 1.0
    fresh = mode == "dense" and not accumulate
    B = inp.B if inp.offsets is not None else 0
    st = tables.backward(dev["grad"], inp.spec.grad_dtype, dev["indices"], dev["offsets"], B,
                         dev["psw"], out, scale=scale, zero_first=fresh)
    torch.cuda.synchronize()
    assert st == "OK", st
    return out0, out.cpu().numpy()


def check_atomic(atomic, inp, mode, accumulate=False, lr=0.01, exact=False):
    out0, got = run_atomic(atomic, inp, mode, accumulate, lr)
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    touched = np.unique(keys)
    elems, valid, _ = row_elements(inp, touched)
    exp, _, _ = expected_rows(inp, touched, mode, out0[elems] if len(touched) else None, None,
                              accumulate, lr, 0.0)
    if len(touched):
        if exact:
            assert np.array_equal(got[elems][valid], np.asarray(exp, np.float32)[valid])
        else:
            assert_close(got[elems], exp, valid, f"atomic {mode}")
    mask = np.ones(got.shape[0], bool)
    mask[elems[valid]] = False
    if mode == "dense" and not accumulate:
        assert np.all(got[mask] == 0)
    else:
        assert np.array_equal(got[mask].view(np.uint32), out0[mask].view(np.uint32))


@pytest.mark.parametrize("mode,accumulate", [("dense", False), ("dense", True), ("sgd", False)])
@pytest.mark.parametrize("pooling,weighted", [("sum", False), ("mean", True)])
def test_atomic_bags(atomic, mode, accumulate, pooling, weighted):
    s = synth.Spec("atomic_bags", 3, (900, 400, 1500), (16, 132, 64), 300, ("uniform", 0, 25),
                   ("zipf", 1.05), pooling, weighted, "f32", mode, seed=41)
    check_atomic(atomic, synth.generate(s), mode, accumulate, lr=0.05)


@pytest.mark.parametrize("D", [64, 1024])
def test_atomic_nobag_bf16(atomic, D):
    s = synth.Spec("atomic_nobag", 1, (3000,), (D,), 0, ("fixed", 1), ("zipf", 1.1), "none", False,
                   "bf16", "dense", accumulate=True, nobag_tokens=2500, seed=D + 1)
    check_atomic(atomic, synth.generate(s), "dense", accumulate=True)


def test_atomic_exact_integer_case(atomic):
    """Small-integer gradients and per-sample weights of 0.5 / 1 / 2: every
    partial sum is exact in fp32, so any order gives the oracle's value."""
    s = synth.Spec("atomic_exact", 2, (50, 70), (8, 12), 64, ("uniform", 0, 12), ("zipf", 1.5),
                   "sum", True, "f32", "dense", seed=5)
    inp = synth.generate(s)
    rng = np.random.default_rng(9)
    inp.grad_output = rng.integers(-8, 9, inp.grad_output.shape).astype(np.float32)
    inp.per_sample_weights = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), inp.N)
    check_atomic(atomic, inp, "dense", exact=True)


def test_atomic_argument_errors(atomic):
    tables = atomic.AtomicTables([0, 10], [0, 8], "none")
    g = torch.zeros(4, 8, device="cuda")
    idx = torch.zeros(4, dtype=torch.int64, device="cuda")
    out = torch.zeros(80, device="cuda")
    w = torch.ones(4, device="cuda")
    # nobag takes no per-sample weights
    assert tables.backward(g, "f32", idx, None, 0, w, out) == "UNSUPPORTED"
    bags = atomic.AtomicTables([0, 10], [0, 8], "sum")
    # bag mode needs offsets and B > 0
    assert bags.backward(g, "f32", idx, None, 4, None, out) == "INVALID_ARGUMENT"
    assert atomic.sgb_atomic_backward(0, None, None, None, 8, 80, "sum", g, "f32", idx, 4, None,
                                      1, None, out, 1.0, 0) == "INVALID_ARGUMENT"
