"""GPU: sgb_backward_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's fixed per-GPU scratch) against
sgb_backward with a caller-allocated workspace, through the C ABI.

Two calls in a row on the shared scratch, the second with a smaller batch of
another shape; each output must equal sgb_backward's bit for bit (the same
kernels, deterministic), which is within the parity tolerance.  A batch that
needs more than the scratch is rejected on the host."""
import sys

import numpy as np
import pytest
import torch

import synth
from harness import to_dev

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


def _buffers(inp, mode, accumulate):
    n = int(inp.weights_offsets[-1])
    if mode == "dense" and not accumulate:
        out0 = np.full(n, np.float32(7.25))
    else:
        out0 = synth.initial_weights(inp)
    mom0 = synth.initial_momentum(inp) if mode == "rowwise_adagrad" else None
    return out0, mom0


def _both(sgb, inp, spec, thr):
    """Outputs of sgb_backward (own workspace) and sgb_backward_noalloc."""
    dev = to_dev(inp)
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, spec.pooling, thr)
    B = inp.B if inp.offsets is not None else 0
    out0, mom0 = _buffers(inp, spec.mode, spec.accumulate)
    res = []
    for noalloc in (False, True):
        out = torch.from_numpy(out0).cuda()
        mom = None if mom0 is None else torch.from_numpy(mom0).cuda()
        kw = dict(grad=out) if spec.mode == "dense" else dict(weights=out, momentum=mom)
        args = (dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], spec.mode)
        opts = dict(accumulate=spec.accumulate, lr=spec.lr or 0.01, eps=spec.eps or 1e-8, **kw)
        if noalloc:
            plan.backward_noalloc(*args, **opts)
            torch.cuda.synchronize()
            status = plan.device_status(None)
        else:
            ws = plan.workspace(inp.N, B)
            plan.backward(*args, workspace=ws, **opts)
            torch.cuda.synchronize()
            status = plan.device_status(ws)
        assert status == "SGB_OK", status
        res.append((out, mom))
    return res


def test_noalloc_matches_backward_two_calls(sgb):
    cases = [
        # larger first: mean pooling with weights, a fresh dense gradient
        synth.spec(2, T=3, E=(20000,) * 3, B=700),
        # then a smaller batch of another shape on the same scratch: row-wise
        # Adagrad over mixed widths with long runs
        synth.spec(3, T=3, E=(3000,) * 3, B=128),
    ]
    for spec in cases:
        inp = synth.generate(spec)
        _say(f"[no-alloc] {spec.name} N={inp.N} mode={spec.mode}")
        (o1, m1), (o2, m2) = _both(sgb, inp, spec, 16)
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "rows differ"
        if m1 is not None:
            assert torch.equal(m1.view(torch.int32), m2.view(torch.int32)), "state differs"


def test_noalloc_rejects_batches_beyond_the_scratch(sgb):
    """About 2.1 M lookups of 128-wide rows need more than the 64 MiB scratch:
    rejected on the host, nothing enqueued."""
    hsc = np.array([0, 20_000_000])
    doff = np.array([0, 128], np.int32)
    plan = sgb.Plan(hsc, doff, "sum", 256)
    N = 2_100_000
    assert plan.workspace_bytes(N, 65536) > (64 << 20)
    idx = torch.zeros(N, dtype=torch.int64, device="cuda")
    off = torch.zeros(65537, dtype=torch.int64, device="cuda")
    g = torch.zeros((65536, 128), dtype=torch.float32, device="cuda")
    w = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(sgb.SgbError) as e:
        plan.backward_noalloc(g, idx, off, 65536, None, "sgd", weights=w, lr=0.1)
    assert e.value.name == "SGB_ERR_WORKSPACE_TOO_SMALL"
