"""GPU test: sgb_backward captured into a HIP graph (torch.cuda.CUDAGraph).

The path enqueues no memsets and allocates nothing, and its fork to the
plan's side streams and the join go through events, which a capture turns
into graph edges.  A captured call is replayed several times, with eager
work and synchronisations between the replays; after every replay the rows
(and momentum) must be bit-equal to the same number of eager calls.  Every
schedule is covered: a small batch runs on the caller's stream alone, larger
ones fork the short-run reduction (and a fresh gradient's zero fill) to the
side streams, right after the sort for rows up to 512 columns, after
run-length encoding for the 1024-column rows.
"""
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


CASES = [
    (dict(cfg=1), "sgd", False),                                   # 301 lookups: one stream
    (dict(cfg=3, T=4, E=(20000,) * 4, B=300), "rowwise_adagrad", False),   # ~24 k: forked
    (dict(cfg=2, T=3, E=(4000, 2500, 3000), B=1500), "dense", False),    # fresh: fill forked too
    (dict(cfg=4, E=(9000,), D=(1024,), nobag_tokens=20000), "dense", True),
    # ~40 k lookups of 64- and 1024-column rows: the early fork, then the
    # wide-row reducer after run-length encoding, on the same side stream
    (dict(cfg=3, T=2, E=(3000, 2000), D=(64, 1024), B=1000), "sgd", False),
]


@pytest.mark.parametrize("ov,mode,acc", CASES)
def test_graph_replays_equal_eager_calls(sgb, ov, mode, acc):
    ov = dict(ov)
    s = synth.spec(ov.pop("cfg"), **ov)
    inp = synth.generate(s)
    dev = to_dev(inp)
    B = inp.B if inp.offsets is not None else 0
    n = int(inp.weights_offsets[-1])
    print(f"[graph] {s.name} {mode} N={inp.N}", flush=True)
    sys.stdout.flush()
    if mode == "dense":
        w0 = torch.from_numpy(synth.initial_weights(inp)).cuda() if acc \
            else torch.full((n,), 7.25, device="cuda")
    else:
        w0 = torch.from_numpy(synth.initial_weights(inp)).cuda()
    m0 = torch.from_numpy(synth.initial_momentum(inp)).cuda() if mode == "rowwise_adagrad" \
        else None
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, s.pooling, 16)
    ws_e, ws_g = plan.workspace(inp.N, B), plan.workspace(inp.N, B)

    def call(w, m, ws, stream=None):
        kw = dict(grad=w) if mode == "dense" else dict(weights=w, momentum=m)
        plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode,
                      accumulate=acc, lr=0.02, eps=1e-6, workspace=ws, stream=stream, **kw)

    we, me = w0.clone(), None if m0 is None else m0.clone()
    wg, mg = w0.clone(), None if m0 is None else m0.clone()
    # one warm-up call on a side stream (scratch copies), then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    wt, mt = w0.clone(), None if m0 is None else m0.clone()
    with torch.cuda.stream(side):
        call(wt, mt, ws_g, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(wg, mg, ws_g, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(wg.view(torch.int32), w0.view(torch.int32)), "the capture ran work"
    for r in range(3):
        graph.replay()
        other = torch.arange(1 << 16, device="cuda", dtype=torch.float32).mul_(0.5)
        call(we, me, ws_e)
        torch.cuda.synchronize()
        assert float(other[2]) == 1.0
        assert plan.device_status(ws_g) == "SGB_OK"
        assert torch.equal(wg.view(torch.int32), we.view(torch.int32)), f"replay {r}: rows"
        if mg is not None:
            assert torch.equal(mg.view(torch.int32), me.view(torch.int32)), f"replay {r}: state"
