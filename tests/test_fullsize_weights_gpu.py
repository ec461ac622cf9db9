"""GPU parity of bf16, fp16 and INT8 weight rows at the full sizes of the
SGD and row-wise Adagrad workloads (configs 1, 3, 5), drawn as bench.py draws
them.

Sampled rows -- the 32 longest runs and 200 random others -- are compared
with the oracle from each row's initial value read back before the call,
with the bounds of the reduced-size tests: bf16 elements within two
roundings plus the fp32 tolerance and at most 1 in 10^3 differing; INT8 codes
within one, at most 1 in 10^3 differing, parameters within 1e-6 + 1e-5 |x|.
2000 sampled untouched rows must be unchanged.
"""
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


def _draw(inp, spec, cfg):
    keys, infos, _ = oracle.linearize(oracle_problem(inp))
    ref = oracle.runs(keys, infos, spec.thr)
    uniq, lens = ref["unique_ids"], ref["run_lengths"]
    rng = np.random.default_rng(100 + cfg)
    top = uniq[np.argsort(-lens, kind="stable")[:32]]
    rnd = rng.choice(uniq, size=min(200, uniq.shape[0]), replace=False)
    sample = np.unique(np.concatenate([top, rnd]))
    untouched = np.setdiff1d(rng.integers(0, inp.total_rows, 4000), uniq)[:2000]
    return sample, untouched


def _momentum(inp, spec):
    if spec.mode != "rowwise_adagrad":
        return None
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed + 1)
    return torch.rand(inp.total_rows, dtype=torch.float32, device="cuda", generator=gen)


def _run(sgb, inp, spec, weights, mom, **kw):
    dev = to_dev(inp)
    B = inp.B if inp.offsets is not None else 0
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, spec.pooling, spec.thr)
    ws = plan.workspace(inp.N, B)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], spec.mode,
                  weights=weights, momentum=mom, lr=spec.lr, eps=spec.eps, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"


def _check_mom(mom, m0s, m0u, sample, untouched, emom, what):
    if mom is None:
        return
    gm = mom[torch.from_numpy(sample).cuda()].cpu().numpy()
    assert_close(gm, emom, None, what + " momentum")
    gmu = mom[torch.from_numpy(untouched).cuda()].cpu().numpy()
    assert np.array_equal(gmu.view(np.uint32), m0u.view(np.uint32))


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_full_size_bf16_rows(sgb, cfg):
    spec = synth.spec(cfg)
    print(f"[fullsize-bf16] config {cfg} {spec.name}: generating", flush=True)
    inp = synth.generate(spec)
    n = int(inp.weights_offsets[-1])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed)
    w = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, spec.weights_std,
                                                                     generator=gen)
    w = w.to(torch.bfloat16)
    mom = _momentum(inp, spec)
    sample, untouched = _draw(inp, spec, cfg)
    elems, valid, D = row_elements(inp, sample)
    uel, uvalid, _ = row_elements(inp, untouched)
    bits = lambda idx: w[torch.from_numpy(idx.reshape(-1)).cuda()].cpu().view(torch.int16) \
        .numpy().view(np.uint16).reshape(idx.shape)
    w0, u0 = bits(elems), bits(uel)
    m0s = None if mom is None else mom[torch.from_numpy(sample).cuda()].cpu().numpy()
    m0u = None if mom is None else mom[torch.from_numpy(untouched).cuda()].cpu().numpy()
    print(f"[fullsize-bf16] config {cfg}: N={inp.N}: run", flush=True)
    _run(sgb, inp, spec, w, mom, stochastic_rounding=True, sr_seed=77, sr_offset=3)
    G, _ = oracle.row_grads(oracle_problem(inp), sample)
    exp, emom = oracle.update_rows_bf16(spec.mode, G, D, np.where(valid, w0, 0), m0s, sample,
                                        lr=spec.lr, eps=spec.eps, stochastic=True, seed=77,
                                        offset=3)
    got = bits(elems)
    diff = (got != exp) & valid
    if diff.any():
        g = (got[diff].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        e = (exp[diff].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(g), np.abs(e)))[1] - 8)
        assert np.all(np.abs(g - e) <= 2 * ulp + 1e-4 + 1e-5 * np.abs(e))
        assert diff.sum() <= max(2, int(valid.sum()) // 1000), f"{int(diff.sum())} differ"
    _check_mom(mom, m0s, m0u, sample, untouched, emom, f"config {cfg}")
    assert np.array_equal(bits(uel)[uvalid], u0[uvalid])
    print(f"[fullsize-bf16] config {cfg}: ok ({int(diff.sum())} one-ulp differences of "
          f"{int(valid.sum())})", flush=True)


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_full_size_int8_rows(sgb, cfg):
    spec = synth.spec(cfg)
    print(f"[fullsize-int8] config {cfg} {spec.name}: generating", flush=True)
    inp = synth.generate(spec)
    E = np.diff(inp.hash_size_cumsum).astype(np.int64)
    Dt = np.diff(inp.D_offsets).astype(np.int64)
    woff8 = np.concatenate([[0], np.cumsum(E * (Dt + 8))]).astype(np.int64)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed + 8)
    w = torch.randint(0, 256, (int(woff8[-1]),), dtype=torch.uint8, device="cuda", generator=gen)
    qp = torch.tensor([0.02 / 255.0, -0.01], dtype=torch.float32, device="cuda").view(torch.uint8)
    for t in range(inp.T):
        w[int(woff8[t]):int(woff8[t + 1])].view(int(E[t]), int(Dt[t]) + 8)[:, int(Dt[t]):] = qp
    mom = _momentum(inp, spec)
    sample, untouched = _draw(inp, spec, cfg)

    def byte_rows(rows):
        t = np.searchsorted(inp.hash_size_cumsum, rows, side="right") - 1
        start = woff8[t] + (rows - inp.hash_size_cumsum[t]) * (Dt[t] + 8)
        cols = np.arange(int(Dt.max()) + 8)[None, :]
        valid = cols < (Dt[t] + 8)[:, None]
        return np.where(valid, start[:, None] + cols, 0), valid, Dt[t]

    idx, valid, D = byte_rows(sample)
    uidx, uvalid, _ = byte_rows(untouched)
    get = lambda i: w[torch.from_numpy(i.reshape(-1)).cuda()].cpu().numpy().reshape(i.shape)
    r0, u0 = get(idx), get(uidx)
    m0s = None if mom is None else mom[torch.from_numpy(sample).cuda()].cpu().numpy()
    m0u = None if mom is None else mom[torch.from_numpy(untouched).cuda()].cpu().numpy()
    print(f"[fullsize-int8] config {cfg}: N={inp.N}: run", flush=True)
    _run(sgb, inp, spec, w, mom)
    G, _ = oracle.row_grads(oracle_problem(inp), sample)
    exp, emom = oracle.update_rows_int8(spec.mode, G, D, np.where(valid, r0, 0), m0s,
                                        lr=spec.lr, eps=spec.eps)
    got = get(idx)
    bad = ncode = 0
    for k in range(sample.shape[0]):
        d = int(D[k])
        gq = got[k, d:d + 8].copy().view(np.float32)
        eq = exp[k, d:d + 8].copy().view(np.float32)
        assert np.all(np.abs(gq - eq) <= 1e-6 + 1e-5 * np.abs(eq)), f"row {sample[k]}: {gq} {eq}"
        dc = np.abs(got[k, :d].astype(int) - exp[k, :d].astype(int))
        assert dc.max() <= 1
        bad += int((dc > 0).sum())
        ncode += d
    assert bad <= max(2, ncode // 1000), f"{bad} of {ncode} codes differ"
    _check_mom(mom, m0s, m0u, sample, untouched, emom, f"config {cfg}")
    assert np.array_equal(get(uidx)[uvalid], u0[uvalid])
    print(f"[fullsize-int8] config {cfg}: ok ({bad} codes off by one of {ncode})", flush=True)


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_full_size_f16_rows(sgb, cfg):
    """fp16 (IEEE binary16) rows with stochastic rounding, as the bf16 case:
    elements within two fp16 spacings plus the fp32 tolerance, at most 1 in
    10^3 differing."""
    spec = synth.spec(cfg)
    print(f"[fullsize-f16] config {cfg} {spec.name}: generating", flush=True)
    inp = synth.generate(spec)
    n = int(inp.weights_offsets[-1])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed)
    w = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, spec.weights_std,
                                                                     generator=gen)
    w = w.to(torch.float16)
    mom = _momentum(inp, spec)
    sample, untouched = _draw(inp, spec, cfg)
    elems, valid, D = row_elements(inp, sample)
    uel, uvalid, _ = row_elements(inp, untouched)
    bits = lambda idx: w[torch.from_numpy(idx.reshape(-1)).cuda()].cpu().view(torch.int16) \
        .numpy().view(np.uint16).reshape(idx.shape)
    w0, u0 = bits(elems), bits(uel)
    m0s = None if mom is None else mom[torch.from_numpy(sample).cuda()].cpu().numpy()
    m0u = None if mom is None else mom[torch.from_numpy(untouched).cuda()].cpu().numpy()
    print(f"[fullsize-f16] config {cfg}: N={inp.N}: run", flush=True)
    _run(sgb, inp, spec, w, mom, stochastic_rounding=True, sr_seed=78, sr_offset=4)
    G, _ = oracle.row_grads(oracle_problem(inp), sample)
    exp, emom = oracle.update_rows_f16(spec.mode, G, D, np.where(valid, w0, 0), m0s, sample,
                                       lr=spec.lr, eps=spec.eps, stochastic=True, seed=78,
                                       offset=4)
    got = bits(elems)
    diff = (got != exp) & valid
    if diff.any():
        g = got[diff].view(np.float16).astype(np.float64)
        e = exp[diff].view(np.float16).astype(np.float64)
        mag = np.maximum(np.abs(g), np.abs(e))
        spacing = np.where(mag < 2.0 ** -14, 2.0 ** -24,
                           np.ldexp(1.0, np.frexp(np.maximum(mag, 2.0 ** -14))[1] - 11))
        assert np.all(np.abs(g - e) <= 2 * spacing + 1e-4 + 1e-5 * np.abs(e))
        assert diff.sum() <= max(2, int(valid.sum()) // 1000), f"{int(diff.sum())} differ"
    _check_mom(mom, m0s, m0u, sample, untouched, emom, f"config {cfg}")
    assert np.array_equal(bits(uel)[uvalid], u0[uvalid])
    print(f"[fullsize-f16] config {cfg}: ok ({int(diff.sum())} one-spacing differences of "
          f"{int(valid.sum())})", flush=True)
