"""Helpers for GPU-vs-oracle parity tests.

Inputs come from `synth` (seeded); expected values come only from `oracle`.
The library is called through its C ABI (the ctypes binding).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import oracle
import synth

ATOL, RTOL = 1e-4, 1e-5   # |gpu - oracle| <= 1e-4 + 1e-5 * |oracle|


def oracle_problem(inp: synth.Inputs) -> oracle.Problem:
    return oracle.problem_from_inputs(inp)


def row_elements(inp: synth.Inputs, rows: np.ndarray):
    """Flat element indices of the given linear rows, and each row's D (padded to max D)."""
    hsc = inp.hash_size_cumsum
    t = np.searchsorted(hsc, rows, side="right") - 1
    D = np.diff(inp.D_offsets).astype(np.int64)[t]
    woff = inp.weights_offsets
    start = woff[t] + (rows - hsc[t]) * D
    Dmax = int(np.max(np.diff(inp.D_offsets)))
    cols = np.arange(Dmax)[None, :]
    valid = cols < D[:, None]
    elems = np.where(valid, start[:, None] + cols, 0)
    return elems, valid, D


@dataclass
class GpuRun:
    out: torch.Tensor              # weights or dense grad after the call (device)
    mom: Optional[torch.Tensor]
    ws: torch.Tensor
    plan: object
    status: str


def to_dev(inp: synth.Inputs):
    g = torch.from_numpy(np.ascontiguousarray(inp.grad_output))
    if inp.grad_output.dtype == np.uint16:
        g = g.view(torch.bfloat16)
    dev = dict(grad=g.cuda(), indices=torch.from_numpy(inp.indices).cuda(),
               offsets=None if inp.offsets is None else torch.from_numpy(inp.offsets).cuda(),
               psw=None if inp.per_sample_weights is None
               else torch.from_numpy(inp.per_sample_weights).cuda())
    return dev


def run_gpu(sgb, inp: synth.Inputs, mode: str, thr: int, out0: torch.Tensor,
            mom0: Optional[torch.Tensor], accumulate=False, lr=0.0, eps=0.0, dev=None,
            plan=None, ws=None) -> GpuRun:
    dev = dev or to_dev(inp)
    plan = plan or sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, thr)
    B = inp.B if inp.offsets is not None else 0
    if ws is None:
        ws = plan.workspace(inp.N, B)
    out = out0.clone()
    mom = None if mom0 is None else mom0.clone()
    kw = dict(weights=out, momentum=mom) if mode != "dense" else dict(grad=out)
    plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], mode,
                  accumulate=accumulate, lr=lr, eps=eps, workspace=ws, **kw)
    torch.cuda.synchronize()
    status = plan.device_status(ws)
    return GpuRun(out, mom, ws, plan, status)


def expected_rows(inp: synth.Inputs, rows: np.ndarray, mode: str, out0_rows: np.ndarray,
                  mom0_rows: Optional[np.ndarray], accumulate=False, lr=0.0, eps=0.0):
    """Oracle value of the given (sorted, distinct) linear rows after the call."""
    G, hits = oracle.row_grads(oracle_problem(inp), rows)
    D = np.diff(inp.D_offsets)[np.searchsorted(inp.hash_size_cumsum, rows, side="right") - 1]
    if mode == "dense" and not accumulate:
        out0_rows = None
    exp, mom = oracle.update_rows(mode, G, D, out0_rows, mom0_rows, lr=lr, eps=eps,
                                  accumulate=accumulate)
    return exp, mom, hits


def assert_close(got: np.ndarray, exp: np.ndarray, valid: Optional[np.ndarray] = None, what=""):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    bad = np.abs(got - exp) > ATOL + RTOL * np.abs(exp)
    if valid is not None:
        bad &= valid
    if bad.any():
        i = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(k)}: gpu={got[tuple(k)]!r} oracle={exp[tuple(k)]!r}" for k in i)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; e.g. {detail}")


def unpack_sorted(view: dict):
    packed = view["sorted_packed"].cpu().numpy().view(np.uint64)
    ib = view["info_bits"]
    keys = (packed >> np.uint64(ib)).astype(np.int64)
    infos = (packed & np.uint64((1 << ib) - 1)).astype(np.int64)
    return keys, infos


def check_runs(sgb, run: GpuRun, inp: synth.Inputs, thr: int):
    """Run structure: bit-exact against the oracle's stable sort and RLE."""
    B = inp.B if inp.offsets is not None else 0
    view = run.plan.runs_view(run.ws, inp.N, B)
    keys, infos, _ = oracle.linearize(oracle_problem(inp))
    ref = oracle.runs(keys, infos, thr)
    gk, gi = unpack_sorted(view)
    assert view["num_runs"] == ref["num_runs"]
    assert np.array_equal(gk, ref["sorted_keys"]), "sorted keys differ"
    assert np.array_equal(gi, ref["sorted_infos"]), "sorted infos differ (stability)"
    assert np.array_equal(view["unique_ids"].cpu().numpy(), ref["unique_ids"])
    assert np.array_equal(view["run_lengths"].cpu().numpy(), ref["run_lengths"])
    assert np.array_equal(view["cumulative"].cpu().numpy(), ref["cumulative"])
    assert view["num_long"] == ref["num_long"]
    assert np.array_equal(view["long_run_ids"].cpu().numpy(), ref["long_run_ids"])
    return ref


def initial_buffers(inp: synth.Inputs, mode: str, accumulate: bool):
    """Host-drawn initial weights / dense grad and momentum, uploaded."""
    n = int(inp.weights_offsets[-1])
    if mode == "dense" and not accumulate:
        # a fresh dense gradient is overwritten: start from garbage to prove it
        out0 = np.full(n, np.float32(7.25))
    else:
        out0 = synth.initial_weights(inp)
    mom0 = synth.initial_momentum(inp) if mode == "rowwise_adagrad" else None
    return out0, mom0


def check_case(sgb, inp: synth.Inputs, mode: str, thr: int, accumulate=False, lr=0.01,
               eps=1e-8, runs=True):
    """Full comparison of every row (small problems)."""
    out0, mom0 = initial_buffers(inp, mode, accumulate)
    d_out0 = torch.from_numpy(out0).cuda()
    d_mom0 = None if mom0 is None else torch.from_numpy(mom0).cuda()
    run = run_gpu(sgb, inp, mode, thr, d_out0, d_mom0, accumulate, lr, eps)
    assert run.status == "SGB_OK", run.status
    got = run.out.cpu().numpy()
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    touched = np.unique(keys)
    elems, valid, _ = row_elements(inp, touched)
    exp, emom, _ = expected_rows(inp, touched, mode, out0[elems] if len(touched) else None,
                                 None if mom0 is None else mom0[touched], accumulate, lr, eps)
    if len(touched):
        assert_close(got[elems], exp, valid, f"{mode} rows")
    # every other element: zero for a fresh dense grad, otherwise bit-unchanged
    mask = np.ones(got.shape[0], bool)
    mask[elems[valid]] = False
    if mode == "dense" and not accumulate:
        assert np.all(got[mask] == 0), "untouched rows of a fresh dense grad must be 0"
    else:
        assert np.array_equal(got[mask].view(np.uint32), out0[mask].view(np.uint32)), \
            "untouched rows changed"
    if mom0 is not None:
        gm = run.mom.cpu().numpy()
        if len(touched):
            assert_close(gm[touched], emom, None, "momentum")
        mm = np.ones(gm.shape[0], bool)
        mm[touched] = False
        assert np.array_equal(gm[mm].view(np.uint32), mom0[mm].view(np.uint32))
    if runs:
        check_runs(sgb, run, inp, thr)
    return run
