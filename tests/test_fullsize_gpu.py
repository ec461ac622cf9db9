"""GPU parity at the five workloads' full sizes, in the configuration bench.py times.

Each workload is drawn exactly as bench.py draws it (same seeds, same plan
and max_segment_length_per_warp) and run once.  Checked against the oracle:
  * the run structure over all N lookups, bit-exact (sorted ids and infos,
    unique ids, run lengths, starts, long runs);
  * every touched row (and, for row-wise Adagrad, every touched momentum
    value) within |gpu - oracle| <= 1e-4 + 1e-5 |oracle|, from the rows'
    initial values read back before the call;
  * every other element of the weights / dense gradient and of the momentum
    bit-unchanged (zero for a fresh dense gradient), compared on the device
    against a copy taken before the call.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, oracle_problem, row_elements, to_dev, unpack_sorted

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sgb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_gradient_backward_amd as m
    return m


def _rows_view(buf, inp, rows):
    """Values of the given linear rows of a flat device buffer, as a padded host array."""
    elems, valid, _ = row_elements(inp, rows)
    idx = torch.from_numpy(elems.reshape(-1)).to(buf.device)
    return buf[idx].cpu().numpy().reshape(elems.shape), valid


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size(sgb, cfg):
    spec = synth.spec(cfg)
    print(f"[fullsize] config {cfg} {spec.name}: generating", flush=True)
    inp = synth.generate(spec)
    dev = to_dev(inp)
    B = inp.B if inp.offsets is not None else 0
    n = int(inp.weights_offsets[-1])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec.seed)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    fresh = spec.mode == "dense" and not spec.accumulate
    if fresh:
        out.fill_(7.25)   # must be overwritten everywhere
    elif spec.mode == "dense":
        out.normal_(0.0, spec.dense_init_std, generator=gen)
    else:
        out.normal_(0.0, spec.weights_std, generator=gen)
    mom = None
    if spec.mode == "rowwise_adagrad":
        mom = torch.rand(inp.total_rows, dtype=torch.float32, device="cuda", generator=gen)

    # oracle run structure (all N lookups); every touched row is compared
    keys, infos, _ = oracle.linearize(oracle_problem(inp))
    ref = oracle.runs(keys, infos, spec.thr)
    uniq, lens = ref["unique_ids"], ref["run_lengths"]
    w0, valid = _rows_view(out, inp, uniq)
    m0 = None if mom is None else mom[torch.from_numpy(uniq).cuda()].cpu().numpy()
    # copies for the untouched check (on the device)
    out0 = out.clone()
    mom_0 = None if mom is None else mom.clone()
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, spec.pooling, spec.thr)
    ws = plan.workspace(inp.N, B)
    kw = dict(grad=out) if spec.mode == "dense" else dict(weights=out, momentum=mom)
    print(f"[fullsize] config {cfg}: N={inp.N} U={ref['num_runs']} long={ref['num_long']}: run",
          flush=True)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], spec.mode,
                  accumulate=spec.accumulate, lr=spec.lr, eps=spec.eps, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert plan.device_status(ws) == "SGB_OK"

    view = plan.runs_view(ws, inp.N, B)
    gk, gi = unpack_sorted(view)
    assert view["num_runs"] == ref["num_runs"] and view["num_long"] == ref["num_long"]
    assert np.array_equal(gk, ref["sorted_keys"])
    assert np.array_equal(gi, ref["sorted_infos"])
    assert np.array_equal(view["unique_ids"].cpu().numpy(), uniq)
    assert np.array_equal(view["run_lengths"].cpu().numpy(), lens)
    assert np.array_equal(view["cumulative"].cpu().numpy(), ref["cumulative"])
    assert np.array_equal(view["long_run_ids"].cpu().numpy(), ref["long_run_ids"])

    G, _ = oracle.row_grads(oracle_problem(inp), uniq)
    D = np.diff(inp.D_offsets)[np.searchsorted(inp.hash_size_cumsum, uniq, side="right") - 1]
    exp, emom = oracle.update_rows(spec.mode, G, D, None if fresh else w0, m0, lr=spec.lr,
                                   eps=spec.eps, accumulate=spec.accumulate)
    del G
    got, _ = _rows_view(out, inp, uniq)
    assert_close(got, exp, valid, f"config {cfg} touched rows")
    del got, exp
    if mom is not None:
        gm = mom[torch.from_numpy(uniq).cuda()].cpu().numpy()
        assert_close(gm, emom, None, f"config {cfg} momentum")
    # every element outside the touched rows: unchanged (zero for a fresh
    # dense gradient), on the device
    elems, _, _ = row_elements(inp, uniq)
    touched_idx = torch.from_numpy(elems[valid]).cuda()
    del elems
    if fresh:
        changed = out.view(torch.int32) != 0
    else:
        changed = out.view(torch.int32) != out0.view(torch.int32)
    changed[touched_idx] = False
    assert not bool(changed.any()), f"config {cfg}: {int(changed.sum())} untouched elements changed"
    del changed, touched_idx, out0
    if mom is not None:
        mchanged = mom.view(torch.int32) != mom_0.view(torch.int32)
        mchanged[torch.from_numpy(uniq).cuda()] = False
        assert not bool(mchanged.any()), "untouched momentum changed"
    print(f"[fullsize] config {cfg}: ok ({uniq.shape[0]} touched rows, {int(valid.sum())} "
          f"elements; all others unchanged)", flush=True)
    sys.stdout.flush()
