#!/usr/bin/env python3
"""Benchmark of the pooled embedding-bag backward on one MI355X.

One step = one sgb_backward() call -- the whole path: linearise, radix sort,
run-length encode, long-run split, segmented reduce and the fused row write
-- over one synthetic batch already resident in HBM.  Default workload: the
largest one that fits one GPU, T=32 tables x E=1M rows with D = 64/128/256
cycling (18.7 GB of weights), B=16384 bags of Poisson(20) lookups drawn
Zipf(1.2), sum pooling, fused row-wise Adagrad; --config selects another one.

Prints ONE JSON line on stdout (progress goes to stderr):
  value        lookups/s of the whole step (wall clock, synchronised)
  achieved_GBps_path   the whole path's algorithmic bytes / step time
  counter_GBps_path    HBM bytes the FETCH_SIZE / WRITE_SIZE counters measured
               for every kernel of the step (profiles/pmc_traffic.txt, when
               taken on the current kernel sources) / step time
  roofline     the dominant kernel (largest time per step): algorithmic bytes
               per launch / its mean launch duration from HIP events around it
  cpu_baseline the CPU oracle (plain C, one thread) on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402  (first: the library binds to torch's HIP runtime)
import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "embedding-bwd lookups/sec + achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
STAGES = ("linearize", "sort_pass", "sort", "rle", "runs", "fill", "reduce_long",
          "reduce_short")
SORT_KERNELS = ("sort_pass",)  # one launch per radix pass, timed on the first pass
KERNEL_SOURCES = ("sparse_gradient_backward_amd/csrc/kernels.hip",
                  "sparse_gradient_backward_amd/csrc/internal.h",
                  "sparse_gradient_backward_amd/csrc/api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def num_cus() -> int:
    """Compute units of the GPU (256 on MI355X when none is visible)."""
    try:
        if torch.cuda.is_available():
            return int(torch.cuda.get_device_properties(0).multi_processor_count)
    except Exception:
        pass
    return 256


def stage_bytes(inp: synth.Inputs, spec: synth.Spec, U: int, run_D: np.ndarray,
                run_len: np.ndarray, thr: int, npasses: int, radix0: int,
                long_rows_D: int | None = None):
    """Algorithmic bytes of one launch of each kernel: every input read once,
    every output written once; a radix pass reads and writes the packed words
    (and coefficients) once; each run's gather and row update once.
    `long_rows_D` (if given) is the sum of D over the grad_output rows the
    long-run reducer reads: it reads a bag's row once for all of the bag's
    lookups of one chunk (see long_gather_elems), so the long runs' gather is
    counted by rows read, not by lookups."""
    N = inp.N
    c = 1 if (spec.pooling == "mean" or spec.weighted) else 0
    sg = 2 if spec.grad_dtype == "bf16" else 4
    BT = inp.B * inp.T if inp.offsets is not None else 0
    rec = 8 + 4 * c                       # packed word (+ coefficient) per lookup
    fresh = spec.mode == "dense" and not spec.accumulate
    Ds = np.diff(inp.D_offsets).astype(np.int64)
    Es = np.diff(inp.hash_size_cumsum).astype(np.int64)
    touched_elems = int(run_D.sum())
    # tiles of the first radix pass (digits of up to 9 bits: 512 x 12 items
    # above 2^22 lookups; above 2^20, 1024 x I with the fewest I in 8..12 that
    # keeps the tiles within the CUs), 512 x 8 above 2^12, else 256 x 8
    if N > (1 << 22) and radix0 <= 512:
        sort_tile = 512 * 12
    elif N > (1 << 20) and radix0 <= 512:
        items = 8
        while items < 12 and (N + 1024 * items - 1) // (1024 * items) > num_cus():
            items += 1
        sort_tile = 1024 * items
    else:
        sort_tile = 512 * 8 if N > (1 << 12) else 256 * 8
    tiles = (N + sort_tile - 1) // sort_tile
    scan_tiles = (N + 4095) // 4096

    def update(D):
        if spec.mode == "dense":
            return int(D.sum()) * 4 * (2 if spec.accumulate else 1)
        if spec.mode == "sgd":
            return int(D.sum()) * 8
        return int(D.sum()) * 8 + D.shape[0] * 8

    lg = run_len >= thr
    gather_long = int((run_len[lg] * run_D[lg]).sum()) * sg
    gather_long_read = gather_long if long_rows_D is None else int(long_rows_D) * sg
    gather_short = int((run_len[~lg] * run_D[~lg]).sum()) * sg
    b = {
        "linearize": N * (8 + 8 + 4 * c + (4 if spec.weighted else 0)) + (BT + 1) * 8 * (BT > 0),
        # a pass reads and writes every packed word (and coefficient) once,
        # its digit totals, and publishes two look-back words per tile and digit
        "sort_pass": N * rec * 2 + tiles * radix0 * 4 * 2 + 8 * radix0 * 4,
        # the sorted words read once (compulsory: beyond 128 tiles the count
        # kernel reads them a second time), two look-back words per tile,
        # each run's unique id, start and run index written
        "rle": N * 8 + scan_tiles * 4 * 2 + U * (8 + 4 + 4),
        "runs": U * (4 + 4) + int(lg.sum()) * (48 + 4 + 4),
        "fill": int((Es * Ds).sum()) * 4 if fresh else 0,
        "reduce_long": gather_long_read + int(run_len[lg].sum()) * rec + int(lg.sum()) * 48
        + update(run_D[lg]),
        "reduce_short": gather_short + N * 8 + int(run_len[~lg].sum()) * 4 * c
        + int((~lg).sum()) * 8 + update(run_D[~lg]),
    }
    b["sort"] = npasses * b["sort_pass"]
    # whole path, counted as the contract's byte model: indices read, the
    # sorted stream (8-byte id + 4-byte info + coefficient) written and read
    # once, the gather, offsets, 24 bytes per run, the row update
    b_path = N * (8 + 2 * (8 + 4 + 4 * c)) + gather_long + gather_short \
        + (BT + 1) * 8 * (BT > 0) + U * 24 + update(run_D)
    if fresh:
        b_path += (int((Es * Ds).sum()) - touched_elems) * 4
    # compulsory bytes: grad_output, indices, offsets and weights read once,
    # the rows updated once (a fresh dense gradient written whole)
    b_comp = int(inp.grad_output.nbytes) + N * 8 + (BT + 1) * 8 * (BT > 0) \
        + (N * 4 if spec.weighted else 0) \
        + (int((Es * Ds).sum()) * 4 if fresh else update(run_D))
    return b, b_path, b_comp


def chunk_len(run_len: np.ndarray, D: np.ndarray, N: int) -> np.ndarray:
    """Lookups per chunk of each long run, as the library cuts them: a base of
    128..512 lookups grown with the batch (one doubling per 2 * 8192 lookups
    above 128 * 8192), divided by the row's 256-column blocks with a floor of
    128, and never more than 1024 chunks per run."""
    base = 128
    while base < 512 and base * 2 * 8192 <= N:
        base *= 2
    cmin = np.maximum(base // ((D + 255) // 256), 128)
    return np.maximum((run_len + 1023) // 1024, cmin)


def lanes_per_row(D: int) -> int:
    """Lanes of a lane group serving a row of D columns at 4 columns per lane:
    the power of two covering D / 4, from 4 to 64."""
    need, lpl = (D + 3) // 4, 4
    while lpl < need and lpl < 64:
        lpl *= 2
    return lpl


def long_gather_elems(sorted_info: np.ndarray, cum: np.ndarray, run_len: np.ndarray,
                      run_D: np.ndarray, thr: int, N: int) -> int:
    """Sum of D over the grad_output rows the long-run reducer reads.  A chunk
    is shared by the 64 / lpl lane groups of a wave in contiguous parts, and
    each group takes its part lpl lookups at a time; within such a slice,
    adjacent lookups of one bag share their grad_output row, which is read
    once (their coefficients are summed first)."""
    lg = np.nonzero(run_len >= thr)[0]
    total = 0
    for r in lg:
        s0, L, D = int(cum[r]), int(run_len[r]), int(run_D[r])
        cl = int(chunk_len(np.array([L]), np.array([D]), N)[0])
        lpl = lanes_per_row(D)
        ng = 64 // lpl
        pos = np.arange(L, dtype=np.int64)
        lo = (pos // cl) * cl
        n = np.minimum(cl, L - lo)
        per = (n + ng - 1) // ng
        off = pos - lo
        within = off - (off // per) * per
        inf = sorted_info[s0:s0 + L]
        new = within % lpl == 0
        new[1:] |= inf[1:] != inf[:-1]
        total += int(new.sum()) * D
    return total


def rle_kernels(N: int) -> str:
    """Kernels of the run-length stage for N sorted positions (tiles of 4096):
    up to 128 tiles the run write alone, up to 4096 the count kernel first,
    beyond that the one-workgroup scan of the counts too."""
    tiles = (N + 4095) // 4096
    if tiles <= 128:
        return "k_rle_write"
    if tiles <= 4096:
        return "k_rle_count+k_rle_write"
    return "k_rle_count+k_rle_scan+k_rle_write"


def short_kernels(dims) -> str:
    """Kernels of the short-run stage: rows up to 512 columns go to the window
    reducer, wider rows to the wide-row reducer."""
    names = []
    if int(np.min(dims)) <= 512:
        names.append("k_reduce_short8")
    if int(np.max(dims)) > 512:
        names.append("k_reduce_wide")
    return "+".join(names)


def kernel_digest() -> str:
    """Short hash of the kernel and launch sources: counter figures taken on
    other sources no longer describe these kernels."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def traffic_table(workload: str) -> dict:
    """HBM bytes per launch of every kernel of one workload, {kernel: (fetch,
    write)}, from the FETCH_SIZE and WRITE_SIZE counter runs recorded in
    profiles/pmc_traffic.txt (already scaled by the copy-kernel calibration);
    empty when no figures exist for the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    src = kernel_digest()
    out = {}
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) < 4 or f[0] != "kernel" or f[1] != workload:
            continue
        # the kernel name may hold spaces ("k_reduce_long[bf16 rows]"): it runs
        # up to the first key=value field
        k = next(i for i, x in enumerate(f) if "=" in x or i == len(f) - 1)
        name = " ".join(f[2:k])
        kv = dict(x.split("=", 1) for x in f[k:] if "=" in x)
        if kv.get("src") == src and "fetch_bytes" in kv and "write_bytes" in kv:
            out[name] = (float(kv["fetch_bytes"]), float(kv["write_bytes"]))
    return out


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of one kernel ('a+b' names sum their kernels), or
    None when the counters were not taken on the current kernel sources."""
    tab = traffic_table(workload)
    parts = kernel.split("+")
    if not all(k in tab for k in parts):
        return None
    return float(sum(sum(tab[k]) for k in parts))


def counter_path_bytes(workload: str, launches: dict):
    """HBM bytes of one whole step by the counters: each path kernel's
    measured bytes per launch times its launches per step (`launches`:
    {kernel: count}); None unless every kernel has a figure for the current
    sources."""
    tab = traffic_table(workload)
    if not launches or not all(k in tab for k in launches):
        return None
    return float(sum(sum(tab[k]) * n for k, n in launches.items()))


def cpu_baseline(inp: synth.Inputs, spec: synth.Spec, thr: int, min_s: float, max_reps: int):
    """The CPU oracle as it stands (plain C, single thread) on the same batch."""
    import oracle
    prob = oracle.problem_from_inputs(inp)
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_s):
        t0 = time.perf_counter()
        keys, infos, _ = oracle.linearize(prob)
        r = oracle.runs(keys, infos, thr)
        G, _ = oracle.row_grads(prob, r["unique_ids"])
        D = np.diff(inp.D_offsets)[np.searchsorted(inp.hash_size_cumsum, r["unique_ids"],
                                                   side="right") - 1]
        rows0 = None if (spec.mode == "dense" and not spec.accumulate) else \
            np.zeros(G.shape, np.float32)
        mom0 = np.zeros(G.shape[0], np.float32) if spec.mode == "rowwise_adagrad" else None
        oracle.update_rows(spec.mode, G, D, rows0, mom0, lr=spec.lr, eps=spec.eps,
                           accumulate=spec.accumulate)
        total += time.perf_counter() - t0
        reps += 1
        log(f"cpu oracle rep {reps}: {total:.1f} s so far")
    return dict(value=inp.N * reps / total, unit="lookups/s", cores=1, kind="oracle",
                sample=f"the full batch ({inp.N} lookups) x {reps} repetition(s), "
                       f"{total:.1f} s, one thread (plain C loops, fp64)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--thr", type=int, default=None,
                    help="max_segment_length_per_warp (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-min-s", type=float, default=10.0)
    ap.add_argument("--cpu-max-reps", type=int, default=2000)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the backward pass here runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)

    import sparse_gradient_backward_amd as sgb
    spec = synth.spec(args.config)
    thr = args.thr or spec.thr
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"config {args.config} ({spec.name}): generating inputs")
    inp = synth.generate(spec)
    g = torch.from_numpy(inp.grad_output)
    if inp.grad_output.dtype == np.uint16:
        g = g.view(torch.bfloat16)
    grad_output = g.to(dev)
    indices = torch.from_numpy(inp.indices).to(dev)
    offsets = None if inp.offsets is None else torch.from_numpy(inp.offsets).to(dev)
    psw = None if inp.per_sample_weights is None else torch.from_numpy(inp.per_sample_weights).to(dev)
    B = inp.B if inp.offsets is not None else 0
    n_elems = int(inp.weights_offsets[-1])
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed)
    out = torch.empty(n_elems, dtype=torch.float32, device=dev)
    mom = None
    if spec.mode == "dense" and not spec.accumulate:
        out.zero_()
    elif spec.mode == "dense":
        out.normal_(0.0, spec.dense_init_std, generator=gen)
    else:
        out.normal_(0.0, spec.weights_std, generator=gen)
    if spec.mode == "rowwise_adagrad":
        mom = torch.zeros(inp.total_rows, dtype=torch.float32, device=dev)   # measurement: state 0
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, spec.pooling, thr)
    ws = plan.workspace(inp.N, B)
    kw = dict(grad=out) if spec.mode == "dense" else dict(weights=out, momentum=mom)
    log(f"N={inp.N} T={inp.T} B={B} workspace={ws.numel() / 2**20:.1f} MiB; warmup {args.warmup}")

    def step(events=None):
        plan.backward(grad_output, indices, offsets, B, psw, spec.mode, accumulate=spec.accumulate,
                      lr=spec.lr, eps=spec.eps, workspace=ws, events=events, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = plan.device_status(ws)
    if status != "SGB_OK":
        raise SystemExit(f"device status after warm-up: {status}")

    # timed region 1: plain steps (the reported value)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # timed region 2: the same steps with HIP events around each kernel,
    # recorded by the library on the stream the kernel runs on (the timed
    # entry point runs the kernels one after another on one stream, so each
    # pair of events brackets one kernel alone)
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(STAGES))]
        for x in e:
            x.record()          # creates the event handle
        evs.append(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms_timed = (time.perf_counter() - t1) * 1e3 / args.steps
    stage_ms = {}  # mean duration of one launch of each kernel ("sort": all passes)
    view = plan.runs_view(ws, inp.N, B)
    for k, name in enumerate(STAGES):
        if name == "fill" and not (spec.mode == "dense" and not spec.accumulate):
            continue
        if name.startswith("sort") and plan_npasses(inp) == 0:
            continue
        d = [e[2 * k].elapsed_time(e[2 * k + 1]) for e in evs]
        stage_ms[name] = float(np.mean(d))
    # cold caches: each call after a 512 MiB write (larger than the L2 caches
    # and the 256 MB MALL), timed by events around the call alone
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
    cold_ev = []
    for _ in range(min(args.steps, 20)):
        flush.fill_(1.0)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        step()
        c1.record()
        cold_ev.append((c0, c1))
    torch.cuda.synchronize()
    cold_ms = float(np.median([c0.elapsed_time(c1) for c0, c1 in cold_ev]))
    del flush
    status = plan.device_status(ws)
    uniq_v = view["unique_ids"].cpu().numpy()
    rows_D = int(np.diff(inp.D_offsets).astype(np.int64)[
        np.searchsorted(inp.hash_size_cumsum, uniq_v, side="right") - 1].sum())
    fwd = forward_measure(plan, inp, spec, indices, offsets, psw, out, ws, args.steps, rows_D)
    piped = pipelined_measure(plan, inp, spec, grad_output, indices, offsets, B, psw, out, mom,
                              args.steps, ms_per_step)
    bf16w = bf16_weights_measure(plan, spec, grad_output, indices, offsets, B, psw, out, mom, ws,
                                 args.steps, ms_per_step)
    f16w = bf16_weights_measure(plan, spec, grad_output, indices, offsets, B, psw, out, mom, ws,
                                args.steps, ms_per_step, dtype=torch.float16)
    int8w = int8_weights_measure(plan, inp, spec, grad_output, indices, offsets, B, psw, mom, ws,
                                 args.steps, ms_per_step)
    atomic = atomic_measure(inp, spec, grad_output, indices, offsets, psw, out,
                            min(args.steps, 20), ms_per_step)

    # run statistics for the byte model (from the library's own run view)
    U = view["num_runs"]
    uniq = view["unique_ids"].cpu().numpy()
    lens = view["run_lengths"].cpu().numpy().astype(np.int64)
    run_t = np.searchsorted(inp.hash_size_cumsum, uniq, side="right") - 1
    run_D = np.diff(inp.D_offsets).astype(np.int64)[run_t]
    nlong = view["num_long"]
    npasses = plan_npasses(inp)
    radix0 = 1 << pass_bits0(inp)
    packed = view["sorted_packed"].cpu().numpy().view(np.uint64)
    infos = (packed & np.uint64((1 << view["info_bits"]) - 1)).astype(np.int64)
    cum = view["cumulative"].cpu().numpy().astype(np.int64)
    long_D = long_gather_elems(infos, cum, lens, run_D, thr, inp.N) \
        if spec.pooling != "none" else None
    del packed, infos
    sb, b_path, b_comp = stage_bytes(inp, spec, U, run_D, lens, thr, npasses, radix0, long_D)
    # the kernel that each stage times ("sort" spans the passes)
    kernel_names = {"reduce_long": "k_reduce_long", "fill": "k_fill", "linearize": "k_linearize",
                    "sort_pass": "k_sort_pass", "rle": rle_kernels(inp.N), "runs": "k_post",
                    "reduce_short": short_kernels(np.diff(inp.D_offsets))}
    # dominant kernel: the largest time per step (a sort kernel runs once per pass)
    per_step = {k: v * (npasses if k in SORT_KERNELS else 1)
                for k, v in stage_ms.items() if k in kernel_names}
    dom = max(per_step, key=lambda k: per_step[k])
    per_launch_bytes = sb[dom]
    per_launch_ms = stage_ms[dom]
    achieved = per_launch_bytes / (per_launch_ms * 1e-3) / 1e9
    gbps_path = b_path / (ms_per_step * 1e-3) / 1e9
    # the whole step by the counters: every kernel of the step, times its
    # launches per step
    launches = {}
    for k, name in kernel_names.items():
        if k not in stage_ms:
            continue
        for kn in name.split("+"):
            launches[kn] = npasses if k in SORT_KERNELS else 1
    cnt_bytes = counter_path_bytes(spec.name, launches)
    cnt_gbps = None if cnt_bytes is None else cnt_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"stages (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))
    log(f"step {ms_per_step:.4f} ms (instrumented {ms_timed:.4f} ms); path {gbps_path:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(inp, spec, thr, args.cpu_min_s, args.cpu_max_reps)

    res = {
        "metric": METRIC,
        "value": inp.N / (ms_per_step * 1e-3),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "T": inp.T, "B": B, "N": inp.N, "U": int(U),
                   "num_long_runs": int(nlong), "max_segment_length_per_warp": thr,
                   "grad_dtype": spec.grad_dtype, "mode": spec.mode,
                   "accumulate": bool(spec.accumulate), "pooling": spec.pooling,
                   "weighted": bool(spec.weighted), "radix_passes": npasses},
        "achieved_GBps_path": gbps_path,
        "hbm_pct_path": 100.0 * gbps_path / HBM_PEAK_GBPS,
        "bytes_alg_path": int(b_path),
        "counter_bytes_path": cnt_bytes,
        "counter_GBps_path": cnt_gbps,
        "hbm_pct_path_counters": None if cnt_gbps is None else 100.0 * cnt_gbps / HBM_PEAK_GBPS,
        "bytes_compulsory": int(b_comp),
        "achieved_GBps_compulsory": b_comp / (ms_per_step * 1e-3) / 1e9,
        "cold": {"ms_per_call_median": cold_ms, "value": inp.N / (cold_ms * 1e-3),
                 "calls": len(cold_ev), "flush_bytes": 512 << 20},
        "stage_ms": stage_ms,
        "stage_bytes": {k: int(v) for k, v in sb.items()},
        "ms_per_step_instrumented": ms_timed,
        "roofline": {"bound": "hbm", "kernel": kernel_names[dom], "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(spec.name, kernel_names[dom]), "bytes_per_launch": int(per_launch_bytes),
                     "launch_ms": per_launch_ms},
        "forward": fwd,
        "pipelined": piped,
        "bf16_weights": bf16w,
        "f16_weights": f16w,
        "int8_weights": int8w,
        "atomic_scatter": atomic,
        "cpu_baseline": cpu,
        "device_status": status,
        "kernel_src": kernel_digest(),
    }
    print(json.dumps(res), flush=True)


def pipelined_measure(plan, inp, spec, grad_output, indices, offsets, B, psw, out, mom, steps,
                      ms_path) -> dict:
    """The same steps through sgb_prepare / sgb_apply, pipelined: the lookups
    of step i+1 are prepared (linearise, sort, runs) into a second workspace
    on one stream while step i is applied (reductions, row updates) on
    another; the applies stay ordered, as updates of one model must. All K
    prepares and K applies are in the timed region (wall clock between two
    synchronisations)."""
    wss = [plan.workspace(inp.N, B), plan.workspace(inp.N, B)]
    # the applies on the current stream, the prepares on one more: with the
    # plan's two side streams that is four, one hardware queue each (more
    # streams than queues would share queues and serialise)
    sf, sm = torch.cuda.Stream(), torch.cuda.current_stream()
    kw = dict(grad=out) if spec.mode == "dense" else dict(weights=out, momentum=mom)
    prepared = [torch.cuda.Event(), torch.cuda.Event()]
    applied = [torch.cuda.Event(), torch.cuda.Event()]

    def run(k):
        sf.wait_stream(sm)
        for e in applied:
            e.record(sm)
        plan.prepare(indices, offsets, B, psw, wss[0], stream=sf)
        prepared[0].record(sf)
        for i in range(k):
            if i + 1 < k:  # the next step's lookups, once its workspace is free
                sf.wait_event(applied[(i + 1) % 2])
                plan.prepare(indices, offsets, B, psw, wss[(i + 1) % 2], stream=sf)
                prepared[(i + 1) % 2].record(sf)
            sm.wait_event(prepared[i % 2])
            plan.apply(grad_output, indices, offsets, B, psw, spec.mode, accumulate=spec.accumulate,
                       lr=spec.lr, eps=spec.eps, workspace=wss[i % 2], stream=sm, **kw)
            applied[i % 2].record(sm)

    run(3)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    status = [plan.device_status(w) for w in wss]
    del wss
    return {"ms_per_step": ms, "value": inp.N / (ms * 1e-3), "steps": steps,
            "vs_plain_step": ms / ms_path,
            "device_status": "SGB_OK" if all(x == "SGB_OK" for x in status) else status}


def forward_measure(plan, inp, spec, indices, offsets, psw, table, ws, steps,
                    rows_D: int) -> dict:
    """The pooled forward (sgb_forward) on the same lookups, reading `table`
    (the workload's weights, or for a dense-gradient workload its gradient
    buffer, which has the weights' shape), timed by HIP events around
    `steps` back-to-back calls.  Its rate is given by compulsory bytes: each
    distinct weight row read once (`rows_D` = the sum of D over the distinct
    rows looked up), the indices (and weights) and offsets read once, the
    output written once; rows looked up again are served by the caches, so
    counting a row per lookup would overstate the HBM rate."""
    B = inp.B if inp.offsets is not None else 0
    doff = inp.D_offsets
    Ds = np.diff(doff).astype(np.int64)
    if spec.pooling == "none":
        shape = (inp.N, int(Ds[0]))
    else:
        shape = (inp.B, int(doff[-1]))
    res = torch.empty(shape, dtype=torch.float32, device=table.device)
    bytes_comp = int(rows_D) * 4 + inp.N * (8 + (4 if inp.per_sample_weights is not None else 0)) \
        + ((B * inp.T + 1) * 8 if inp.offsets is not None else 0) + int(np.prod(shape)) * 4

    def call():
        plan.forward(indices, offsets, B, psw, table, res, ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    status = plan.device_status(ws)
    gbps = bytes_comp / (ms * 1e-3) / 1e9
    return {"ms_per_call": ms, "lookups_per_s": inp.N / (ms * 1e-3),
            "bytes_compulsory": int(bytes_comp), "device_status": status,
            "roofline": {"bound": "hbm", "kernel": "k_forward", "achieved": gbps,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                         "bytes": "compulsory",
                         "traffic": measured_traffic(spec.name, "k_forward")}}


def bf16_weights_measure(plan, spec, grad_output, indices, offsets, B, psw, out, mom, ws, steps,
                         ms_path, dtype=torch.bfloat16):
    """The same step with the weights held in a 16-bit type (bf16, or fp16
    with dtype=torch.float16) and stochastic rounding in the fused update
    (SGD and row-wise Adagrad workloads only): a 16-bit copy of the weights
    (nearest-even of the fp32 ones), `steps` plain calls timed by HIP
    events, each with its own Philox offset."""
    if spec.mode == "dense":
        return None
    w = out.to(dtype)
    m = None if mom is None else mom.clone()

    def call(k):
        plan.backward(grad_output, indices, offsets, B, psw, spec.mode, weights=w, momentum=m,
                      lr=spec.lr, eps=spec.eps, workspace=ws, stochastic_rounding=True,
                      sr_seed=spec.seed, sr_offset=k)

    for k in range(3):
        call(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        call(3 + k)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    status = plan.device_status(ws)
    del w, m
    return {"ms_per_step": ms, "stochastic_rounding": True, "vs_fp32_weights": ms / ms_path,
            "device_status": status}


def int8_weights_measure(plan, inp, spec, grad_output, indices, offsets, B, psw, mom, ws, steps,
                         ms_path):
    """The same step with INT8 row-wise quantized weight rows (SGD and
    row-wise Adagrad workloads): synthetic rows
    made on the device (codes uniform in [0, 255], scale 0.02 / 255, bias
    -0.01, so values span [-0.01, 0.01]), `steps` plain calls timed by HIP
    events."""
    D = np.diff(inp.D_offsets).astype(np.int64)
    if spec.mode == "dense":
        return None
    E = np.diff(inp.hash_size_cumsum).astype(np.int64)
    woff8 = np.concatenate([[0], np.cumsum(E * (D + 8))])
    dev = grad_output.device
    g = torch.Generator(device=dev)
    g.manual_seed(spec.seed + 8)
    w = torch.randint(0, 256, (int(woff8[-1]),), dtype=torch.uint8, device=dev, generator=g)
    qp = torch.tensor([0.02 / 255.0, -0.01], dtype=torch.float32, device=dev).view(torch.uint8)
    for t in range(inp.T):
        rows = w[int(woff8[t]):int(woff8[t + 1])].view(int(E[t]), int(D[t]) + 8)
        rows[:, int(D[t]):] = qp
    m = None if mom is None else mom.clone()

    def call():
        plan.backward(grad_output, indices, offsets, B, psw, spec.mode, weights=w, momentum=m,
                      lr=spec.lr, eps=spec.eps, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    status = plan.device_status(ws)
    del w, m
    return {"ms_per_step": ms, "vs_fp32_weights": ms / ms_path, "device_status": status}


def atomic_measure(inp, spec, grad_output, indices, offsets, psw, out, calls, ms_path) -> dict:
    """The atomic scatter-add baseline (libsgb_atomic.so: every lookup adds
    its bag's gradient row into the looked-up row with fp32 atomics, no
    deduplication) on the same lookups, timed by HIP events around `calls`
    back-to-back calls.  Dense workloads produce the same dense gradient
    (fresh or accumulated); SGD and row-wise Adagrad workloads are run as
    atomic SGD on the same weights (row-wise Adagrad has no atomic form).
    Runs after every other measurement: it changes `out`."""
    import sparse_gradient_backward_amd.atomic as atomic
    tables = atomic.AtomicTables(inp.hash_size_cumsum, inp.D_offsets, spec.pooling)
    B = inp.B if inp.offsets is not None else 0
    dense = spec.mode == "dense"
    mode = "dense" if dense else "sgd"
    scale = 1.0 if dense else -(spec.lr or 0.01)
    fresh = dense and not spec.accumulate

    def call():
        return tables.backward(grad_output, spec.grad_dtype, indices, offsets, B, psw, out,
                               scale=scale, zero_first=fresh)

    st = call()
    torch.cuda.synchronize()
    if st != "OK":
        return {"status": st}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    return {"mode": mode, "accumulate": bool(not fresh) if dense else None, "calls": calls,
            "ms_per_call": ms, "lookups_per_s": inp.N / (ms * 1e-3),
            "float_atomics_per_call": int(np.diff(inp.D_offsets).astype(np.int64)[
                np.repeat(np.arange(inp.T), np.diff(inp.offsets[::inp.B]))
                if inp.offsets is not None else np.zeros(inp.N, np.int64)].sum()),
            "slowdown_vs_path": ms / ms_path, "status": st}


def plan_npasses(inp: synth.Inputs) -> int:
    rows = int(inp.hash_size_cumsum[-1])
    bits = int(rows - 1).bit_length()
    return (bits + 9) // 10


def pass_bits0(inp: synth.Inputs) -> int:
    """Digit bits of the first radix pass (the library splits the id bits evenly)."""
    rows = int(inp.hash_size_cumsum[-1])
    bits = int(rows - 1).bit_length()
    n = plan_npasses(inp)
    return bits // n + (1 if bits % n else 0) if n else 0


if __name__ == "__main__":
    main()
