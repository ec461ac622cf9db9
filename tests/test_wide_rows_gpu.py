"""GPU parity of the whole-row updates on rows wider than 1024 columns:
row-wise Adagrad on fp32 and bf16 rows, and INT8 rows under SGD and row-wise
Adagrad, at D = 2048, 4096 and 8192 in one plan.

The mean square (Adagrad) and the requantization range (INT8) need the whole
row before any element is written, so these rows are served in passes over
their 256-column blocks: short runs by a wave that gathers the run again on
each pass, long runs by the chunked reducer whose last wave reads the summed
partials again on each pass.  thr = 4 sends the hot runs to the chunked
reducer; thr = 2^31 - 1 leaves every run short.  Tolerances as for the other
row kinds (see test_bf16_gpu and test_int8_gpu)."""
import sys

import pytest
import torch

import synth
from harness import check_case
from test_bf16_gpu import check_bf16
from test_int8_gpu import check_int8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sgb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_gradient_backward_amd as m
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def wide_spec(mode, grad_dtype="f32", seed=71):
    # three tables of 2048, 4096 and 8192 columns; Zipf ids make runs of
    # 1 to a few hundred lookups
    return synth.Spec("wide_rows", 3, (300, 200, 100), (2048, 4096, 8192), 48,
                      ("uniform", 1, 14), ("zipf", 1.3), "sum", True, grad_dtype, mode,
                      lr=0.02, eps=1e-6, seed=seed)


THRS = [4, 2**31 - 1]


@pytest.mark.parametrize("thr", THRS)
@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_wide_adagrad_fp32_rows(sgb, thr, grad_dtype):
    inp = synth.generate(wide_spec("rowwise_adagrad", grad_dtype))
    _say(f"[wide] adagrad fp32 rows thr={thr} grad={grad_dtype} N={inp.N}")
    check_case(sgb, inp, "rowwise_adagrad", thr, lr=0.02, eps=1e-6)


@pytest.mark.parametrize("thr", THRS)
def test_wide_sgd_and_dense_rows(sgb, thr):
    """The dense and SGD paths on the same wide rows (any width was served
    before; kept beside the whole-row cases)."""
    inp = synth.generate(wide_spec("sgd"))
    _say(f"[wide] sgd fp32 rows thr={thr} N={inp.N}")
    check_case(sgb, inp, "sgd", thr, lr=0.02)


@pytest.mark.parametrize("thr", THRS)
@pytest.mark.parametrize("stochastic", [True, False])
def test_wide_adagrad_bf16_rows(sgb, thr, stochastic):
    inp = synth.generate(wide_spec("rowwise_adagrad", seed=73))
    _say(f"[wide] adagrad bf16 rows thr={thr} sr={stochastic} N={inp.N}")
    check_bf16(sgb, inp, "rowwise_adagrad", thr, stochastic)


@pytest.mark.parametrize("thr", THRS)
@pytest.mark.parametrize("mode", ["sgd", "rowwise_adagrad"])
def test_wide_int8_rows(sgb, thr, mode):
    inp = synth.generate(wide_spec(mode, seed=79))
    _say(f"[wide] int8 rows {mode} thr={thr} N={inp.N}")
    check_int8(sgb, inp, mode, thr)
