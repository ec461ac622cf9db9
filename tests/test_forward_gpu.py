"""GPU parity of the pooled forward (sgb_forward) against the oracle.

Inputs come from `synth` (seeded) with seeded weights; expected values only
from `oracle.forward`.  Reduced-size cases compare every output element;
full-size workloads compare sampled bags (or lookups without bags), each
sample checked by the oracle on a sub-problem made of exactly the sampled
bags and the weight rows they read.  Tolerance as for the backward:
|gpu - oracle| <= 1e-4 + 1e-5 |oracle|.  The output is pre-filled with NaN,
so an element the kernel does not write fails.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close

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


def _problem(inp):
    return oracle.Problem(T=inp.T, B=inp.B, hash_size_cumsum=inp.hash_size_cumsum,
                          D_offsets=inp.D_offsets, offsets=inp.offsets, indices=inp.indices,
                          per_sample_weights=inp.per_sample_weights, pooling=inp.spec.pooling,
                          grad_output=None)


def _out_shape(inp):
    doff = inp.D_offsets
    if inp.spec.pooling == "none":
        return (inp.N, int(doff[1] - doff[0]))
    return (inp.B, int(doff[-1]))


def _run(sgb, inp, W, plan=None, ws=None):
    plan = plan or sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, 256)
    B = inp.B if inp.offsets is not None else 0
    ind = torch.from_numpy(inp.indices).cuda()
    off = None if inp.offsets is None else torch.from_numpy(inp.offsets).cuda()
    psw = None if inp.per_sample_weights is None else torch.from_numpy(inp.per_sample_weights).cuda()
    out = torch.full(_out_shape(inp), float("nan"), dtype=torch.float32, device="cuda")
    ws = plan.workspace(inp.N, B) if ws is None else ws
    plan.forward(ind, off, B, psw, W, out, ws)
    torch.cuda.synchronize()
    return out, plan.device_status(ws)


def _weights_np(inp, seed):
    return np.random.default_rng(seed).standard_normal(int(inp.weights_offsets[-1])).astype(np.float32)


def check_forward(sgb, inp, seed=0, what=""):
    Wn = _weights_np(inp, seed)
    out, st = _run(sgb, inp, torch.from_numpy(Wn).cuda())
    assert st == "SGB_OK", st
    exp = oracle.forward(_problem(inp), Wn)
    assert_close(out.cpu().numpy(), exp, None, what)


CASES = {
    "c1": (1, dict()),
    "c2": (2, dict(T=3, E=(20000,) * 3, B=700)),
    "c3": (3, dict(T=6, E=(30000,) * 6, B=900)),
    "c4": (4, dict(E=(9000,), D=(512,), nobag_tokens=6000)),
    "c5": (5, dict(E=(200000,), B=1500)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_config_shaped(sgb, name):
    cfg, kw = CASES[name]
    inp = synth.generate(synth.spec(cfg, **kw))
    _say(f"[forward] {name} N={inp.N} T={inp.T} B={inp.B}")
    check_forward(sgb, inp, seed=cfg, what=name)


@pytest.mark.parametrize("pooling,weighted", [("sum", False), ("sum", True), ("mean", False),
                                              ("mean", True)])
@pytest.mark.parametrize("D", [4, 12, 64, 256, 1024, 4096])
def test_forward_widths(sgb, pooling, weighted, D):
    s = synth.Spec("fw", 1, (500,), (D,), 37, ("uniform", 0, 9), ("zipf", 1.1), pooling, weighted,
                   "f32", "dense", seed=D)
    inp = synth.generate(s)
    check_forward(sgb, inp, seed=3, what=f"D={D} {pooling} w={weighted}")


def test_forward_mixed_widths(sgb):
    """Tables of different width: lane groups sized for the narrowest."""
    s = synth.Spec("fmix", 4, (50, 700, 90, 300), (4, 68, 256, 1024), 53, ("uniform", 0, 12),
                   ("zipf", 1.05), "mean", True, "f32", "dense", seed=5)
    check_forward(sgb, synth.generate(s), seed=4, what="mixed widths")


@pytest.mark.parametrize("D", [16, 128, 4096])
def test_forward_nobag(sgb, D):
    s = synth.Spec("fnb", 1, (3000,), (D,), 0, ("fixed", 1), ("zipf", 1.1), "none", False,
                   "f32", "dense", nobag_tokens=1029, seed=D + 1)
    check_forward(sgb, synth.generate(s), seed=5, what=f"nobag D={D}")


def test_forward_nobag_multi_table_offsets(sgb):
    s = synth.Spec("fnb2", 3, (40, 70, 25), (32, 32, 32), 11, ("uniform", 0, 6), ("uniform",),
                   "none", False, "f32", "dense", seed=17)
    check_forward(sgb, synth.generate(s), seed=6, what="nobag with offsets")


def test_forward_empty_bags(sgb):
    s = synth.Spec("femp", 2, (30, 40), (8, 16), 64, ("uniform", 0, 1), ("uniform",), "mean",
                   False, "f32", "dense", seed=19)
    inp = synth.generate(s)
    check_forward(sgb, inp, seed=7, what="mostly empty bags")
    none = synth.generate(s)
    none.indices = none.indices[:0]
    none.offsets = np.zeros_like(none.offsets)
    Wn = _weights_np(none, 8)
    out, st = _run(sgb, none, torch.from_numpy(Wn).cuda())
    assert st == "SGB_OK"
    assert torch.all(out == 0)


def test_forward_errors(sgb):
    s = synth.Spec("ferr", 2, (30, 40), (8, 8), 20, ("uniform", 1, 5), ("uniform",), "sum", False,
                   "f32", "dense", seed=10)
    inp = synth.generate(s)
    W = torch.from_numpy(_weights_np(inp, 1)).cuda()
    bad = synth.generate(s)
    bad.indices = bad.indices.copy()
    bad.indices[inp.offsets[20] + 1] = 40          # table 1 has E = 40
    assert _run(sgb, bad, W)[1] == "SGB_ERR_INDEX_OUT_OF_RANGE"
    bad = synth.generate(s)
    bad.offsets = bad.offsets.copy()
    bad.offsets[5], bad.offsets[6] = bad.offsets[6], bad.offsets[5] - 1
    assert _run(sgb, bad, W)[1] == "SGB_ERR_BAD_OFFSETS"
    bad = synth.generate(s)
    bad.offsets = bad.offsets.copy()
    bad.offsets[-1] -= 1
    assert _run(sgb, bad, W)[1] == "SGB_ERR_BAD_OFFSETS"
    assert _run(sgb, inp, W)[1] == "SGB_OK"
    # host-detected: weighted nobag is unsupported, a misaligned output is rejected
    nb = synth.Spec("ferr2", 1, (30,), (8,), 0, ("fixed", 1), ("uniform",), "none", False, "f32",
                    "dense", nobag_tokens=10, seed=12)
    ni = synth.generate(nb)
    plan = sgb.Plan(ni.hash_size_cumsum, ni.D_offsets, "none", 256)
    ind = torch.from_numpy(ni.indices).cuda()
    Wn = torch.from_numpy(_weights_np(ni, 2)).cuda()
    out = torch.empty((10, 8), device="cuda")
    ws = plan.workspace(10, 0)
    with pytest.raises(sgb.SgbError) as e:
        plan.forward(ind, None, 0, torch.ones(10, device="cuda"), Wn, out, ws)
    assert e.value.name == "SGB_ERR_UNSUPPORTED"
    with pytest.raises(sgb.SgbError) as e:
        plan.forward(ind, None, 0, None, Wn, torch.empty(81, device="cuda")[1:].view(10, 8), ws)
    assert e.value.name == "SGB_ERR_INVALID_ARGUMENT"


def test_forward_adjoint_of_gpu_backward(sgb):
    """<forward(W), G> == <W, dense backward(G)> with both GPU paths."""
    s = synth.Spec("fadj", 3, (400, 900, 300), (16, 64, 32), 120, ("uniform", 0, 14),
                   ("zipf", 1.1), "mean", True, "f32", "dense", seed=23)
    inp = synth.generate(s)
    Wn = _weights_np(inp, 9)
    W = torch.from_numpy(Wn).cuda()
    out, st = _run(sgb, inp, W)
    assert st == "SGB_OK"
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, "mean", 8)
    ws = plan.workspace(inp.N, inp.B)
    grad = torch.zeros_like(W)
    G = torch.from_numpy(inp.grad_output).cuda()
    plan.backward(G, torch.from_numpy(inp.indices).cuda(), torch.from_numpy(inp.offsets).cuda(),
                  inp.B, torch.from_numpy(inp.per_sample_weights).cuda(), "dense", grad=grad,
                  workspace=ws)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"
    lhs = float((out.double() * G.double()).sum())
    rhs = float((W.double() * grad.double()).sum())
    assert abs(lhs - rhs) <= 1e-5 * (abs(lhs) + abs(rhs)) + 1e-5, (lhs, rhs)


def _sub_problem(inp, t, bags):
    """The sampled bags of table t as a problem of their own: one table made of
    the rows they read (remapped in order of first use), and those rows' ids."""
    off = inp.offsets
    B = inp.B
    lo = [int(off[t * B + b]) for b in bags]
    hi = [int(off[t * B + b + 1]) for b in bags]
    idx = np.concatenate([inp.indices[a:c] for a, c in zip(lo, hi)]) if bags else np.zeros(0, np.int64)
    rows, inv = np.unique(idx, return_inverse=True)
    if rows.size == 0:
        rows = np.zeros(1, np.int64)
    D = int(inp.D_offsets[t + 1] - inp.D_offsets[t])
    sub_off = np.concatenate([[0], np.cumsum(np.array(hi) - np.array(lo))]).astype(np.int64)
    psw = None
    if inp.per_sample_weights is not None:
        psw = np.concatenate([inp.per_sample_weights[a:c] for a, c in zip(lo, hi)]).astype(np.float32)
    p = oracle.Problem(T=1, B=len(bags), hash_size_cumsum=np.array([0, rows.size]),
                       D_offsets=np.array([0, D]), offsets=sub_off, indices=inv.astype(np.int64),
                       per_sample_weights=psw, pooling=inp.spec.pooling, grad_output=None)
    return p, rows, D


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_forward_full_size(sgb, cfg):
    spec = synth.spec(cfg)
    _say(f"[forward-full] config {cfg} {spec.name}: generating")
    inp = synth.generate(spec)
    n = int(inp.weights_offsets[-1])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed + 7)
    W = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=gen)
    out, st = _run(sgb, inp, W)
    assert st == "SGB_OK", st
    rng = np.random.default_rng(cfg)
    doff = inp.D_offsets
    if inp.spec.pooling == "none":
        D = int(doff[1])
        look = np.unique(rng.integers(0, inp.N, 300))
        rows = np.unique(inp.indices[look])
        inv = np.searchsorted(rows, inp.indices[look])
        Wr = W.view(-1, D)[torch.from_numpy(rows).cuda()].cpu().numpy()
        p = oracle.Problem(T=1, B=0, hash_size_cumsum=np.array([0, rows.size]),
                           D_offsets=np.array([0, D]), offsets=None, indices=inv.astype(np.int64),
                           per_sample_weights=None, pooling="none", grad_output=None)
        exp = oracle.forward(p, Wr.reshape(-1))
        got = out[torch.from_numpy(look).cuda()].cpu().numpy()
        assert_close(got, exp, None, f"config {cfg} sampled lookups")
        return
    lens = np.diff(inp.offsets).reshape(inp.T, inp.B)
    checked = 0
    for t in range(inp.T):
        bags = set(rng.choice(inp.B, size=min(inp.B, max(4, 200 // inp.T)), replace=False).tolist())
        bags |= set(np.argsort(-lens[t], kind="stable")[:4].tolist())   # the longest bags
        bags = sorted(int(b) for b in bags)
        p, rows, D = _sub_problem(inp, t, bags)
        w0 = int(inp.weights_offsets[t])
        el = (w0 + rows[:, None] * D + np.arange(D)[None, :]).reshape(-1)
        Wr = W[torch.from_numpy(el).cuda()].cpu().numpy()
        exp = oracle.forward(p, Wr)
        c0 = int(doff[t])
        got = out[torch.from_numpy(np.array(bags)).cuda(), c0:c0 + D].cpu().numpy()
        assert_close(got, exp, None, f"config {cfg} table {t} sampled bags")
        checked += len(bags)
    _say(f"[forward-full] config {cfg}: ok ({checked} bags)")
