"""GPU parity: the HIP path through the C ABI against the CPU oracle.

fp32 results: |gpu - oracle| <= 1e-4 + 1e-5 |oracle| per element; integer
run structure (sorted ids and infos, unique ids, run lengths, starts, long
runs): bit-exact; untouched rows: bit-unchanged (zero for a fresh dense grad).
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import synth
import oracle
from harness import (assert_close, check_case, check_runs, expected_rows, initial_buffers,
                     oracle_problem, row_elements, run_gpu, to_dev)

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


def small_spec(cfg, **kw):
    """A configuration's shape and distributions at a size the oracle finishes quickly."""
    return synth.spec(cfg, **kw)


# configuration-shaped cases at reduced size (several tiles + ragged tails)
CASES = {
    "c1": (1, dict()),
    "c2": (2, dict(T=3, E=(20000,) * 3, B=700)),
    "c3": (3, dict(T=6, E=(30000,) * 6, B=900)),
    "c4": (4, dict(E=(9000,), D=(512,), nobag_tokens=6000)),
    "c5": (5, dict(E=(200000,), B=1500)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_config_shaped(sgb, name):
    cfg, kw = CASES[name]
    s = small_spec(cfg, **kw)
    inp = synth.generate(s)
    _say(f"[parity] {name} N={inp.N} T={inp.T} B={inp.B} mode={s.mode}")
    check_case(sgb, inp, s.mode, s.thr, accumulate=s.accumulate, lr=s.lr or 0.01,
               eps=s.eps or 1e-8)


@pytest.mark.parametrize("thr", [1, 2, 63, 64, 65, 2**31 - 1])
def test_thresholds(sgb, thr):
    s = synth.Spec("thr", 2, (300, 50), (64, 16), 40, ("uniform", 0, 70), ("zipf", 1.5), "sum",
                   True, "f32", "rowwise_adagrad", lr=0.05, eps=1e-6, seed=500 + thr % 97)
    inp = synth.generate(s)
    _say(f"[parity] thr={thr} N={inp.N}")
    check_case(sgb, inp, "rowwise_adagrad", thr, lr=0.05, eps=1e-6)


SWEEP = []
for T in (1, 3):
    for B in (1, 7, 64):
        for pooling, weighted in (("sum", False), ("sum", True), ("mean", False), ("mean", True)):
            for mode in ("dense", "sgd", "rowwise_adagrad"):
                SWEEP.append((T, B, pooling, weighted, mode))


@pytest.mark.parametrize("T,B,pooling,weighted,mode", SWEEP)
def test_sweep(sgb, T, B, pooling, weighted, mode):
    Ds = (4, 12, 64, 132, 256)
    D = tuple(Ds[(t + B + (3 if weighted else 0)) % len(Ds)] for t in range(T))
    E = tuple(5 + 37 * (t + 1) for t in range(T))
    seed = zlib.crc32(repr((T, B, pooling, weighted, mode)).encode()) % 100000
    s = synth.Spec("sweep", T, E, D, B, ("uniform", 0, 70), ("zipf", 1.1), pooling, weighted,
                   "f32", mode, seed=seed)
    inp = synth.generate(s)
    acc = mode == "dense" and B % 2 == 1
    check_case(sgb, inp, mode, 16, accumulate=acc, lr=0.03, eps=1e-7)


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [4, 64, 256, 1024, 4096])
def test_nobag(sgb, grad_dtype, D):
    s = synth.Spec("nobag", 1, (3000,), (D,), 0, ("fixed", 1), ("zipf", 1.1), "none", False,
                   grad_dtype, "dense", accumulate=True, nobag_tokens=2500, seed=D)
    inp = synth.generate(s)
    check_case(sgb, inp, "dense", 128, accumulate=True)


def test_nobag_multi_table_offsets(sgb):
    s = synth.Spec("nobag2", 3, (500, 70, 900), (32, 32, 32), 50, ("uniform", 0, 9),
                   ("uniform",), "none", False, "bf16", "dense", seed=31)
    inp = synth.generate(s, with_grad=False)
    inp.grad_output = synth.bf16_bits(
        inp.rngs["grad_output"].standard_normal((inp.N, 32), dtype=np.float32))
    check_case(sgb, inp, "dense", 8, accumulate=False)


def test_wide_rows_adagrad_and_sgd(sgb):
    for mode in ("rowwise_adagrad", "sgd", "dense"):
        s = synth.Spec("wide", 2, (400, 300), (1024, 516), 33, ("uniform", 0, 40), ("zipf", 1.3),
                       "mean", True, "f32", mode, seed=77)
        check_case(sgb, synth.generate(s), mode, 32, lr=0.02, eps=1e-6)


def test_wide_and_narrow_tables_all_short(sgb):
    """Rows wider than 512 columns beside narrow ones; a threshold above every
    run length sends even the hottest runs (hundreds of lookups, several
    64-lookup slices) through the short-run reducers."""
    s = synth.Spec("widemix", 3, (700, 500, 300), (64, 2048, 772), 257, ("uniform", 0, 30),
                   ("zipf", 1.2), "sum", True, "bf16", "dense", seed=91)
    inp = synth.generate(s)
    check_case(sgb, inp, "dense", 2**31 - 1, accumulate=False)
    check_case(sgb, inp, "sgd", 2**31 - 1, lr=0.05)
    check_case(sgb, inp, "dense", 40, accumulate=True)


@pytest.mark.parametrize("mode,acc", [("dense", True), ("dense", False), ("sgd", False),
                                      ("rowwise_adagrad", False)])
def test_medium_runs_of_wide_rows(sgb, mode, acc):
    """Medium runs of wide rows: runs of 1 to 257 lookups (63/64/65 and
    255/256/257 among them) in tables of 512, 2048 and 4096 columns, thr =
    256.  The runs below 256 lookups of the two wider tables are each gathered
    by the wave of one (run, column block) item of the wide-row reducer, those
    of the 512-column table by the window reducer; from 256 on the chunked
    long-run reducer serves them, and they form the long-run list."""
    lens = np.array([1, 63, 64, 65, 200, 255, 256, 257, 2, 31])
    B = int(lens.sum())
    s = synth.Spec("medium", 3, (64, 64, 64), (512, 2048, 4096), B, ("fixed", 1), ("uniform",),
                   "sum", False, "bf16", mode, accumulate=acc, seed=53)
    inp = synth.generate(s)
    rng = np.random.default_rng(54)
    parts = []
    for _ in range(3):
        ids = rng.choice(64, size=lens.shape[0], replace=False)
        v = np.repeat(ids, lens)
        rng.shuffle(v)
        parts.append(v)
    inp.indices = np.concatenate(parts).astype(np.int64)
    _say(f"[parity] medium runs of wide rows {mode} acc={acc} N={inp.N}")
    check_case(sgb, inp, mode, 256, accumulate=acc, lr=0.05, eps=1e-6)


@pytest.mark.parametrize("T", [512, 600])
@pytest.mark.parametrize("mode", ["dense", "sgd", "rowwise_adagrad"])
def test_many_tables(sgb, T, mode):
    """Run post-processing stages the table metadata in LDS for up to 512
    tables and reads it from memory beyond that; the reducers read it through
    scalar loads indexed by table: 512 and 600 tables of 8, 64, 520 and 1028
    columns, Zipf ids so that some runs are long (thr = 4)."""
    dims = tuple((8, 64, 520, 1028)[t % 4] for t in range(T))
    s = synth.Spec("manytables", T, (40,) * T, dims, 24, ("uniform", 0, 5), ("zipf", 1.3),
                   "sum", False, "f32", mode, seed=83)
    inp = synth.generate(s)
    _say(f"[parity] {T} tables {mode} N={inp.N}")
    check_case(sgb, inp, mode, 4, lr=0.02, eps=1e-6)


def _early_fork_case(seed):
    """Three tables of 64, 256 and 1024 columns, 9001 one-lookup bags each
    (27 003 lookups: above the single-stream limit, a ragged last window).
    Each table's runs have lengths that sit around the 64-position windows
    and the thresholds below (1 .. 4097 lookups, the largest id of each
    table 100), the rest of its bags runs of 1 to 5 lookups, ids shuffled so
    that the runs fall at every offset of a window."""
    B = 9001
    s = synth.Spec("earlyfork", 3, (20000, 20000, 20000), (64, 256, 1024), B, ("fixed", 1),
                   ("uniform",), "sum", False, "f32", "sgd", seed=seed)
    inp = synth.generate(s)
    rng = np.random.default_rng(seed)
    fixed = [1, 2, 63, 64, 65, 127, 128, 129, 130, 200, 1000]
    cols = []
    for t in range(3):
        lens = [4095 + t] + (list(fixed) if t == 0 else list(rng.choice(fixed, 6, replace=False)))
        while B - 100 - sum(lens) > 5:
            lens.append(int(rng.integers(1, 6)))
        if B - 100 - sum(lens) > 0:
            lens.append(B - 100 - sum(lens))
        ids = rng.choice(19999, size=len(lens), replace=False)
        v = np.concatenate([np.repeat(ids, lens), np.full(100, 19999)])
        assert v.size == B
        rng.shuffle(v)
        cols.append(v)
    inp.indices = np.concatenate(cols).astype(np.int64)
    return inp


@pytest.mark.parametrize("thr", [1, 64, 129, 4096, 4097])
def test_early_fork_run_scan(sgb, thr):
    """Batches between the single-stream limit and 2^22 lookups, with a
    long-run threshold of at most 4096, start the short-run reducer of rows
    up to 512 columns right after the sort: it finds the length of each
    window's last run by scanning the sorted words after the window (up to
    thr words past the run's head), while run-length encoding and the
    long-run list run beside it; the 1024-column rows' reducer waits for the
    run starts.  thr = 4097 takes the fork after run-length encoding."""
    inp = _early_fork_case(61)
    _say(f"[parity] early fork thr={thr} N={inp.N}")
    check_case(sgb, inp, "sgd", thr, lr=0.05)


@pytest.mark.parametrize("mode,acc", [("dense", False), ("dense", True), ("rowwise_adagrad", False)])
def test_early_fork_modes(sgb, mode, acc):
    """The early fork with a fresh dense gradient (the side stream also waits
    for the zero fill), an accumulated one, and row-wise Adagrad."""
    inp = _early_fork_case(62)
    _say(f"[parity] early fork {mode} acc={acc} N={inp.N}")
    check_case(sgb, inp, mode, 129, accumulate=acc, lr=0.05, eps=1e-6)


@pytest.mark.parametrize("mode,acc,thr", [("sgd", False, 129), ("dense", False, 64),
                                          ("dense", True, 4096)])
def test_early_fork_equals_serial_schedule(sgb, mode, acc, thr):
    """The early fork (run lengths from the sorted ids after each window,
    rows up to 512 columns reduced beside run-length encoding, the
    1024-column rows after it) gives bit-identical rows to the timed entry
    point, which runs every kernel in order on one stream and takes the run
    lengths from the run starts."""
    inp = _early_fork_case(63)
    _say(f"[parity] early fork vs serial {mode} acc={acc} thr={thr} N={inp.N}")
    dev = to_dev(inp)
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, inp.spec.pooling, thr)
    ws = plan.workspace(inp.N, inp.B)
    o0, m0 = initial_buffers(inp, mode, acc)
    outs = []
    for timed in (False, True):
        out = torch.from_numpy(o0).cuda()
        kw = dict(grad=out) if mode == "dense" else dict(weights=out, momentum=None)
        events = None
        if timed:
            events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sgb.STAGES))]
            for e in events:
                e.record()
        plan.backward(dev["grad"], dev["indices"], dev["offsets"], inp.B, dev["psw"], mode,
                      accumulate=acc, lr=0.05, eps=1e-6, workspace=ws, events=events, **kw)
        torch.cuda.synchronize()
        assert plan.device_status(ws) == "SGB_OK"
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_wide_rows_more_items_than_waves(sgb):
    """~50 000 runs of 2048-column rows: ~200 000 (run, column block) items,
    more than the wide-row reducer's waves (sixteen times the resident
    workgroups), so waves take a second item after their first."""
    s = synth.Spec("wideloop", 1, (80000,), (2048,), 0, ("fixed", 1), ("uniform",), "none", False,
                   "bf16", "dense", accumulate=True, nobag_tokens=80000, seed=43)
    inp = synth.generate(s)
    _say(f"[parity] wide rows, many items N={inp.N}")
    check_case(sgb, inp, "dense", 64, accumulate=True)
    check_case(sgb, inp, "dense", 64, accumulate=False)


# ------------------------------------------------------------------ edge cases

def test_empty_input(sgb):
    s = synth.Spec("empty", 2, (10, 20), (8, 16), 5, ("fixed", 0), ("uniform",), "sum", False,
                   "f32", "dense", seed=1)
    inp = synth.generate(s)
    assert inp.N == 0
    for mode, acc in (("dense", False), ("dense", True), ("sgd", False), ("rowwise_adagrad", False)):
        check_case(sgb, inp, mode, 4, accumulate=acc, runs=False)


def test_all_empty_but_one(sgb):
    s = synth.Spec("one", 2, (50, 60), (16, 32), 100, ("fixed", 0), ("uniform",), "mean", True,
                   "f32", "sgd", seed=2)
    inp = synth.generate(s, with_grad=True)
    lens = np.zeros(200, np.int64)
    lens[137] = 9
    inp.offsets = np.concatenate([[0], np.cumsum(lens)])
    inp.indices = np.array([3, 3, 59, 0, 3, 7, 7, 1, 3])
    inp.per_sample_weights = np.linspace(0.5, 2.0, 9).astype(np.float32)
    check_case(sgb, inp, "sgd", 2)


def test_one_hot_row(sgb):
    """Every lookup on one row: one run of length N, long path only."""
    s = synth.Spec("hot", 1, (1000,), (128,), 3000, ("uniform", 1, 40), ("uniform",), "sum", True,
                   "f32", "rowwise_adagrad", seed=3)
    inp = synth.generate(s)
    inp.indices[:] = 417
    _say(f"[parity] one row N={inp.N}")
    check_case(sgb, inp, "rowwise_adagrad", 64, lr=0.01, eps=1e-8)
    check_case(sgb, inp, "dense", 64)


def test_all_distinct(sgb):
    """U = N, short path only."""
    B = 5000
    s = synth.Spec("distinct", 1, (B,), (64,), B, ("fixed", 1), ("uniform",), "mean", False, "f32",
                   "dense", seed=4)
    inp = synth.generate(s)
    inp.indices = np.random.default_rng(5).permutation(B).astype(np.int64)
    check_case(sgb, inp, "dense", 2)


@pytest.mark.parametrize("delta", [-1, 0, 1])
def test_run_lengths_around_threshold(sgb, delta):
    thr = 64
    L = thr + delta
    s = synth.Spec("around", 1, (50,), (16,), 3 * L, ("fixed", 1), ("uniform",), "sum", False,
                   "f32", "sgd", seed=6)
    inp = synth.generate(s)
    inp.indices = np.repeat(np.array([5, 9, 40]), L).astype(np.int64)
    check_case(sgb, inp, "sgd", thr)


def test_mixed_dims_and_bf16_bags(sgb):
    s = synth.Spec("mixed", 4, (700, 20, 1500, 90), (8, 200, 48, 132), 300, ("poisson", 6.0),
                   ("zipf", 1.2), "mean", True, "bf16", "rowwise_adagrad", lr=0.1, eps=1e-5,
                   seed=8)
    check_case(sgb, synth.generate(s), "rowwise_adagrad", 24, lr=0.1, eps=1e-5)


def test_huge_run_two_level_combine(sgb):
    """A run long enough for several first-level groups of chunks."""
    s = synth.Spec("huge", 1, (100,), (64,), 8000, ("uniform", 20, 40), ("zipf", 3.0), "sum",
                   True, "f32", "rowwise_adagrad", lr=0.01, eps=1e-8, seed=9)
    inp = synth.generate(s)
    _say(f"[parity] huge run N={inp.N}")
    check_case(sgb, inp, "rowwise_adagrad", 64, lr=0.01, eps=1e-8)


@pytest.mark.parametrize("tokens", [300_000, 128 * 4096, 128 * 4096 + 1, 4096 * 4096,
                                    4096 * 4096 + 1])
def test_many_run_tiles(sgb, tokens):
    """Run-length tiles of 4096 sorted positions: up to 128 tiles the run
    write alone (look-back over the tile counts), up to 4096 the count kernel
    and a run write that sums the counts itself, beyond that the scan kernel
    too; each limit and one more.  Runs are compared bit-exact, rows to the
    usual tolerance."""
    s = synth.Spec("tiles", 1, (60000,), (4,), 0, ("fixed", 1), ("zipf", 1.05), "none", False,
                   "f32", "dense", accumulate=True, nobag_tokens=tokens, seed=41)
    inp = synth.generate(s)
    _say(f"[parity] many run tiles N={inp.N}")
    check_case(sgb, inp, "dense", 64, accumulate=True)


SORT_SHAPES = [
    # (rows, lookups, index distribution): id bits -> digits per radix pass; tile shape
    (1, 3000, ("uniform",)),            # 0 bits: nothing to sort
    (2, 4000, ("uniform",)),            # 1 bit, radix 2 (most look-back lanes idle); small tiles
    (6, 4096, ("zipf", 1.5)),           # 3 bits, radix 8; small tiles, the largest such batch
    (60000, 4097, ("zipf", 1.05)),      # 16 bits -> 8/8; medium tiles from here
    (60000, 65537, ("zipf", 1.05)),     # 17 medium tiles
    (1 << 20, 300_000, ("uniform",)),   # 20 bits -> 10/10: medium tiles with 1024 digits
    (1 << 20, 1_200_000, ("zipf", 1.1)),  # 10-bit digits keep medium tiles above 2^20 lookups
    # large tiles of 1024 x I items, I the fewest of 8..12 that keeps the
    # tiles within the CUs (on a 256-CU GPU: I = 8 up to 2^21 lookups, 9 up
    # to 2.36 M, 10 up to 2.62 M, 11 up to 2.88 M, then 12)
    (1 << 22, 1_200_000, ("zipf", 1.2)),  # 22 bits -> 8/7/7: 1024 x 8, skewed ids
    ((1 << 25) - 1, 1_500_000, ("uniform",)),  # 25 bits -> 9/8/8: 1024 x 8
    ((1 << 25) - 1, (1 << 21) + 1, ("zipf", 1.2)),  # 1024 x 9
    ((1 << 25) - 1, 2_500_000, ("uniform",)),  # 1024 x 10
    ((1 << 25) - 1, 2_800_000, ("zipf", 1.1)),  # 1024 x 11
    ((1 << 25) - 1, 1 << 22, ("uniform",)),    # 1024 x 12, the largest batch of large tiles
    ((1 << 25) - 1, (1 << 22) + 1, ("zipf", 1.2)),  # huge tiles (683) from here
    (1 << 20, (1 << 22) + 1, ("uniform",)),    # 10-bit digits keep medium tiles
]


@pytest.mark.parametrize("rows,tokens,dist", SORT_SHAPES)
def test_sort_shapes(sgb, rows, tokens, dist):
    """Every radix tile shape and digit width of the single-sweep passes
    (look-back over up to several hundred tiles, histograms counted by the
    linearisation and by each pass for the next): the run structure is
    compared bit-exact, rows to the usual tolerance."""
    s = synth.Spec("sortshape", 1, (rows,), (4,), 0, ("fixed", 1), dist, "none", False,
                   "f32", "dense", accumulate=True, nobag_tokens=tokens, seed=61 + rows % 89)
    inp = synth.generate(s)
    _say(f"[parity] sort shape rows={rows} N={inp.N} dist={dist}")
    check_case(sgb, inp, "dense", 64, accumulate=True)


def test_runs_view_rejects_another_layout(sgb):
    """The run view needs the N and B of the last call on the workspace
    (they fix its layout); the call records them, and a view asked with
    other sizes is refused instead of pointing into the wrong regions."""
    s = synth.spec(1)
    inp = synth.generate(s)
    out0, _ = initial_buffers(inp, s.mode, False)
    run = run_gpu(sgb, inp, s.mode, 4, torch.from_numpy(out0).cuda(), None, lr=s.lr)
    assert run.status == "SGB_OK"
    v = run.plan.runs_view(run.ws, inp.N, inp.B)
    assert v["num_runs"] > 0
    for N, B in ((inp.N - 1, inp.B), (inp.N, inp.B + 1)):
        with pytest.raises(sgb.SgbError) as e:
            run.plan.runs_view(run.ws, N, B)
        assert e.value.name == "SGB_ERR_INVALID_ARGUMENT"


# ------------------------------------------------------------------ properties

def test_deterministic(sgb):
    s = synth.spec(5, E=(50000,), B=3000)
    inp = synth.generate(s)
    out0, mom0 = initial_buffers(inp, s.mode, False)
    d0, m0 = torch.from_numpy(out0).cuda(), torch.from_numpy(mom0).cuda()
    dev = to_dev(inp)
    r1 = run_gpu(sgb, inp, s.mode, 64, d0, m0, lr=s.lr, eps=s.eps, dev=dev)
    r2 = run_gpu(sgb, inp, s.mode, 64, d0, m0, lr=s.lr, eps=s.eps, dev=dev, plan=r1.plan)
    assert torch.equal(r1.out.view(torch.int32), r2.out.view(torch.int32))
    assert torch.equal(r1.mom.view(torch.int32), r2.mom.view(torch.int32))


def test_workspace_reuse_smaller_second_call(sgb):
    """The same workspace serves a big call and then a smaller one."""
    s1 = synth.spec(3, T=3, E=(5000,) * 3, B=600)
    s2 = synth.spec(3, T=3, E=(5000,) * 3, B=200, seed=77)
    plan = sgb.Plan(synth.generate(s1).hash_size_cumsum, synth.generate(s1).D_offsets, "sum", 32)
    inp1, inp2 = synth.generate(s1), synth.generate(s2)
    ws = plan.workspace(max(inp1.N, inp2.N), 600)
    for inp in (inp1, inp2):
        out0, mom0 = initial_buffers(inp, "rowwise_adagrad", False)
        run = run_gpu(sgb, inp, "rowwise_adagrad", 32, torch.from_numpy(out0).cuda(),
                      torch.from_numpy(mom0).cuda(), lr=0.01, eps=1e-8, plan=plan, ws=ws)
        assert run.status == "SGB_OK"
        check_runs(sgb, run, inp, 32)


# ------------------------------------------------------------------ errors

def test_device_detected_errors(sgb):
    s = synth.Spec("err", 2, (30, 40), (8, 8), 20, ("uniform", 1, 5), ("uniform",), "sum", False,
                   "f32", "dense", seed=10)
    inp = synth.generate(s)
    out0 = torch.zeros(int(inp.weights_offsets[-1]), device="cuda")
    bad = synth.generate(s)
    bad.indices = bad.indices.copy()
    bad.indices[inp.offsets[20] + 1] = 40          # table 1 has E = 40: out of range
    r = run_gpu(sgb, bad, "dense", 4, out0, None)
    assert r.status == "SGB_ERR_INDEX_OUT_OF_RANGE"
    bad = synth.generate(s)
    bad.indices = bad.indices.copy()
    bad.indices[0] = -3
    assert run_gpu(sgb, bad, "dense", 4, out0, None).status == "SGB_ERR_INDEX_OUT_OF_RANGE"
    bad = synth.generate(s)
    bad.offsets = bad.offsets.copy()
    bad.offsets[5], bad.offsets[6] = bad.offsets[6], bad.offsets[5] - 1
    assert run_gpu(sgb, bad, "dense", 4, out0, None).status == "SGB_ERR_BAD_OFFSETS"
    bad = synth.generate(s)
    bad.offsets = bad.offsets.copy()
    bad.offsets[-1] -= 1
    assert run_gpu(sgb, bad, "dense", 4, out0, None).status == "SGB_ERR_BAD_OFFSETS"
    # a clean call on the same plan afterwards is fine again
    assert run_gpu(sgb, inp, "dense", 4, out0, None).status == "SGB_OK"


def test_host_detected_errors(sgb):
    s = synth.Spec("herr", 1, (30,), (8,), 4, ("uniform", 1, 5), ("uniform",), "none", False,
                   "f32", "dense", seed=11)
    with pytest.raises(sgb.SgbError) as e:
        sgb.Plan(np.array([0, 10]), np.array([0, 6]), "sum", 4)
    assert e.value.name == "SGB_ERR_INVALID_ARGUMENT"
    with pytest.raises(sgb.SgbError):
        sgb.Plan(np.array([0, 10, 10]), np.array([0, 8, 16]), "sum", 4)
    with pytest.raises(sgb.SgbError):
        sgb.Plan(np.array([0, 10]), np.array([0, 8]), "sum", 0)
    plan = sgb.Plan(np.array([0, 10]), np.array([0, 8]), "none", 4)
    idx = torch.zeros(4, dtype=torch.int64, device="cuda")
    g = torch.zeros(4, 8, device="cuda")
    grad = torch.zeros(80, device="cuda")
    ws = plan.workspace(4, 0)
    with pytest.raises(sgb.SgbError) as e:   # nobag is unweighted only
        plan.backward(g, idx, None, 0, torch.ones(4, device="cuda"), "dense", grad=grad,
                      workspace=ws)
    assert e.value.name == "SGB_ERR_UNSUPPORTED"
    with pytest.raises(sgb.SgbError) as e:
        plan.backward(g, idx, None, 0, None, "dense", grad=grad, workspace=ws[:16])
    assert e.value.name == "SGB_ERR_WORKSPACE_TOO_SMALL"
    with pytest.raises(sgb.SgbError) as e:
        plan.backward(g, idx, None, 0, None, "sgd", workspace=ws)   # no weights
    assert e.value.name == "SGB_ERR_INVALID_ARGUMENT"


@pytest.mark.parametrize("cfg", [2, 5])
def test_own_stream_and_timed(sgb, cfg):
    """The call on a stream of the caller's own, completed by synchronising that
    stream alone (the side streams are joined back into it), matches the
    oracle; the timed entry point (events around every kernel, every kernel
    on the one stream, run lengths from the run starts) gives bit-identical
    outputs to the plain call (here, for both workloads, with the short-run
    reducer forked right after the sort and, for the dense one, the zero
    fill forked at the start)."""
    s = synth.spec(2, T=2, E=(4000, 3000), B=700) if cfg == 2 else \
        synth.spec(5, E=(60000,), B=2000)
    inp = synth.generate(s)
    _say(f"[parity] own stream config {cfg} N={inp.N}")
    dev = to_dev(inp)
    plan = sgb.Plan(inp.hash_size_cumsum, inp.D_offsets, s.pooling, 64)
    B = inp.B
    ws = plan.workspace(inp.N, B)
    o0, m0h = initial_buffers(inp, s.mode, s.accumulate)
    out0 = torch.from_numpy(o0).cuda()
    mom0 = None if m0h is None else torch.from_numpy(m0h).cuda()
    outs = []
    for timed in (False, True):
        out = out0.clone()
        mom = None if mom0 is None else mom0.clone()
        kw = dict(weights=out, momentum=mom) if s.mode != "dense" else dict(grad=out)
        st = torch.cuda.Stream()
        torch.cuda.synchronize()
        events = None
        if timed:
            events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sgb.STAGES))]
            with torch.cuda.stream(st):
                for e in events:
                    e.record()
        with torch.cuda.stream(st):
            plan.backward(dev["grad"], dev["indices"], dev["offsets"], B, dev["psw"], s.mode,
                          accumulate=s.accumulate, lr=s.lr, eps=s.eps, workspace=ws,
                          stream=st, events=events, **kw)
        st.synchronize()  # only this stream
        host = out.cpu().numpy()
        outs.append((host, None if mom is None else mom.cpu().numpy()))
        assert plan.device_status(ws, st) == "SGB_OK"
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    if outs[0][1] is not None:
        assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    # and the values are the oracle's
    keys, _, _ = oracle.linearize(oracle_problem(inp))
    rows = np.unique(keys)
    elems, valid, _ = row_elements(inp, rows)
    m0 = None if m0h is None else m0h[rows]
    exp, emom, _ = expected_rows(inp, rows, s.mode, o0[elems], m0, accumulate=s.accumulate,
                                 lr=s.lr, eps=s.eps)
    assert_close(outs[0][0][elems], exp, valid, "rows on the caller's stream")
