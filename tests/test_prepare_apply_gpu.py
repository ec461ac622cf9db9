"""GPU tests of the two-part entry points sgb_prepare / sgb_apply.

* prepare then apply on one stream is the same computation as sgb_backward:
  outputs and momentum bit-equal to a backward call on the same inputs, and
  the run structure (after prepare alone) bit-exact against the oracle;
* the pipelined use the split exists for -- the next batch prepared into a
  second workspace on another stream while the current batch is applied --
  gives bit-equal rows to the same batches applied one backward call after
  another (row-wise Adagrad and SGD on shared weights, so the applies must
  stay ordered), and the result agrees with the oracle;
* host-detected errors of the two entry points.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (assert_close, check_runs, expected_rows, initial_buffers, row_elements,
                     to_dev, GpuRun)

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


CASES = [
    # (spec overrides, mode, accumulate)
    (dict(cfg=2, T=3, E=(4000, 2500, 3000), B=300), "dense", False),
    (dict(cfg=4, E=(9000,), D=(1024,), nobag_tokens=5000), "dense", True),
    (dict(cfg=3, T=4, E=(20000,) * 4, B=500), "rowwise_adagrad", False),
    (dict(cfg=5, E=(60000,), B=800), "rowwise_adagrad", False),
    (dict(cfg=1), "sgd", False),
]


def _spec(ov):
    ov = dict(ov)
    return synth.spec(ov.pop("cfg"), **ov)


@pytest.mark.parametrize("ov,mode,acc", CASES)
def test_prepare_apply_equals_backward(sgb, ov, mode, acc):
    s = _spec(ov)
    inp = synth.generate(s)
    dev = to_dev(inp)
    B = inp.B if inp.offsets is not None else 0
    thr = 16
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, s.pooling, thr)
    out0, mom0 = initial_buffers(inp, mode, acc)
    d_out0 = torch.from_numpy(out0).cuda()
    d_mom0 = None if mom0 is None else torch.from_numpy(mom0).cuda()
    _say(f"[prepare/apply] {s.name} {mode} N={inp.N}")

    def kw(out, mom):
        return dict(weights=out, momentum=mom) if mode != "dense" else dict(grad=out)

    # one backward call
    ws1 = plan.workspace(inp.N, B)
    out1, mom1 = d_out0.clone(), None if d_mom0 is None else d_mom0.clone()
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode,
                  accumulate=acc, lr=s.lr, eps=s.eps, workspace=ws1, **kw(out1, mom1))
    # prepare, check the run structure it left, then apply
    ws2 = plan.workspace(inp.N, B)
    out2, mom2 = d_out0.clone(), None if d_mom0 is None else d_mom0.clone()
    plan.prepare(dev["indices"], dev["offsets"], B, dev["psw"], ws2)
    torch.cuda.synchronize()
    assert plan.device_status(ws2) == "SGB_OK"
    check_runs(sgb, GpuRun(None, None, ws2, plan, "SGB_OK"), inp, thr)
    plan.apply(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode,
               accumulate=acc, lr=s.lr, eps=s.eps, workspace=ws2, **kw(out2, mom2))
    torch.cuda.synchronize()
    assert plan.device_status(ws1) == "SGB_OK" and plan.device_status(ws2) == "SGB_OK"
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), "rows differ"
    if mom1 is not None:
        assert torch.equal(mom1.view(torch.int32), mom2.view(torch.int32)), "momentum differs"


@pytest.mark.parametrize("mode", ["rowwise_adagrad", "sgd"])
def test_pipelined_batches(sgb, mode):
    """Three batches of one table set applied to one set of weights: batch
    i+1 is prepared on a second stream into the other workspace while batch
    i is applied; the applies stay ordered on the first stream."""
    specs = [synth.spec(3, T=4, E=(20000,) * 4, B=400, seed=300 + k) for k in range(3)]
    inps = [synth.generate(sp) for sp in specs]
    devs = [to_dev(x) for x in inps]
    s0 = specs[0]
    B = s0.B
    thr = 16
    plan = sgb.Plan(inps[0].hash_size_cumsum, inps[0].D_offsets, s0.pooling, thr)
    out0, mom0 = initial_buffers(inps[0], mode, False)
    d_out0 = torch.from_numpy(out0).cuda()
    d_mom0 = None if mom0 is None else torch.from_numpy(mom0).cuda()
    nmax = max(x.N for x in inps)
    lr, eps = 0.02, 1e-6

    def kw(out, mom):
        return dict(weights=out, momentum=mom)

    # sequential reference: one backward call per batch
    ws = plan.workspace(nmax, B)
    out_s, mom_s = d_out0.clone(), None if d_mom0 is None else d_mom0.clone()
    for x, d in zip(inps, devs):
        plan.backward(d["grad"], d["indices"], d["offsets"], B, d["psw"], mode, lr=lr, eps=eps,
                      workspace=ws, **kw(out_s, mom_s))
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"

    # pipelined: prepares on stream F (two workspaces), applies on stream M
    wss = [plan.workspace(nmax, B), plan.workspace(nmax, B)]
    out_p, mom_p = d_out0.clone(), None if d_mom0 is None else d_mom0.clone()
    sf, sm = torch.cuda.Stream(), torch.cuda.Stream()
    sf.wait_stream(torch.cuda.current_stream())
    sm.wait_stream(torch.cuda.current_stream())
    prepared = [torch.cuda.Event() for _ in range(3)]
    applied = [torch.cuda.Event() for _ in range(3)]
    # host order matters: an event is waited for only after it has been
    # recorded, so batch i + 1 is prepared in the same iteration as batch i
    # is applied, and batch i + 1 reuses the workspace of batch i - 1 only
    # after that batch's apply has been recorded
    plan.prepare(devs[0]["indices"], devs[0]["offsets"], B, devs[0]["psw"], wss[0], stream=sf)
    prepared[0].record(sf)
    for i, d in enumerate(devs):
        if i + 1 < len(devs):
            n = devs[i + 1]
            if i >= 1:
                sf.wait_event(applied[i - 1])
            plan.prepare(n["indices"], n["offsets"], B, n["psw"], wss[(i + 1) % 2], stream=sf)
            prepared[i + 1].record(sf)
        sm.wait_event(prepared[i])
        plan.apply(d["grad"], d["indices"], d["offsets"], B, d["psw"], mode, lr=lr, eps=eps,
                   workspace=wss[i % 2], stream=sm, **kw(out_p, mom_p))
        applied[i].record(sm)
    torch.cuda.current_stream().wait_stream(sm)
    torch.cuda.synchronize()
    assert plan.device_status(wss[0]) == "SGB_OK" and plan.device_status(wss[1]) == "SGB_OK"
    assert torch.equal(out_s.view(torch.int32), out_p.view(torch.int32)), "rows differ"
    if mom_s is not None:
        assert torch.equal(mom_s.view(torch.int32), mom_p.view(torch.int32)), "momentum differs"

    # and against the oracle, batch after batch on the host
    rows_all = np.unique(np.concatenate([oracle.linearize(oracle.problem_from_inputs(x))[0]
                                         for x in inps]))
    elems, valid, _ = row_elements(inps[0], rows_all)
    w = out0[elems]
    m = None if mom0 is None else mom0[rows_all]
    for x in inps:
        keys = np.unique(oracle.linearize(oracle.problem_from_inputs(x))[0])
        sel = np.searchsorted(rows_all, keys)
        exp, emom, _ = expected_rows(x, keys, mode, w[sel], None if m is None else m[sel],
                                     lr=lr, eps=eps)
        w[sel] = np.where(valid[sel], exp, w[sel])
        if m is not None:
            m[sel] = emom
    got = out_p.cpu().numpy()[elems]
    assert_close(got, w, valid, f"pipelined {mode} rows")
    if m is not None:
        assert_close(mom_p.cpu().numpy()[rows_all], m, None, "pipelined momentum")


def test_prepare_apply_errors(sgb):
    s = synth.spec(1)
    inp = synth.generate(s)
    dev = to_dev(inp)
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, s.pooling, 4)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sgb.SgbError) as e:
        plan.prepare(dev["indices"], dev["offsets"], inp.B, dev["psw"], small)
    assert e.value.status == sgb.SGB_ERR_WORKSPACE_TOO_SMALL
    out = torch.from_numpy(synth.initial_weights(inp)).cuda()
    with pytest.raises(sgb.SgbError) as e:
        plan.apply(dev["grad"], dev["indices"], dev["offsets"], inp.B, dev["psw"], "sgd",
                   weights=out, lr=0.1, workspace=small)
    assert e.value.status == sgb.SGB_ERR_WORKSPACE_TOO_SMALL
    ws = plan.workspace(inp.N, inp.B)
    with pytest.raises(sgb.SgbError) as e:  # SGD needs weights
        plan.apply(dev["grad"], dev["indices"], dev["offsets"], inp.B, dev["psw"], "sgd",
                   lr=0.1, workspace=ws)
    assert e.value.status == sgb.SGB_ERR_INVALID_ARGUMENT


def test_apply_on_a_workspace_prepared_for_other_lookups(sgb):
    """sgb_apply checks on the device that the workspace's run structure is
    that of its own lookups (the header records the N and B of the prepare
    that wrote it): with other sizes the reducers do nothing and the call
    reports SGB_ERR_INTERNAL; the rows stay as they were."""
    s1 = synth.spec(3, T=3, E=(5000,) * 3, B=300, seed=401)
    s2 = synth.spec(3, T=3, E=(5000,) * 3, B=300, seed=402)
    i1, i2 = synth.generate(s1), synth.generate(s2)
    assert i1.N != i2.N
    d1, d2 = to_dev(i1), to_dev(i2)
    plan = sgb.Plan(i1.hash_size_cumsum, i1.D_offsets, s1.pooling, 16)
    ws = plan.workspace(max(i1.N, i2.N), s1.B)
    w = torch.from_numpy(synth.initial_weights(i1)).cuda()
    w0 = w.clone()
    plan.prepare(d1["indices"], d1["offsets"], s1.B, d1["psw"], ws)
    plan.apply(d2["grad"], d2["indices"], d2["offsets"], s2.B, d2["psw"], "sgd", weights=w,
               lr=0.1, workspace=ws)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_ERR_INTERNAL"
    assert torch.equal(w.view(torch.int32), w0.view(torch.int32))
