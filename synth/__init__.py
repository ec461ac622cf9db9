"""Seeded synthetic inputs for the pooled embedding-bag backward.

This module only *draws inputs* (bag lengths, row indices, output gradients,
per-sample weights, initial weights/state).  It computes nothing of the
backward method itself, so both the GPU tests and the CPU oracle may take
their inputs from here.

Workloads (the five configurations of the contract):
  1  T=1, E=1000, D=16, weights N(0, 0.01); B=64, L ~ U[0, 8]; uniform ids;
     sum pooling; fp32 grad N(0, 1); SGD lr=0.01.
  2  T=8, E=100000 each, D=128; B=2048, L ~ U[1, 32]; Zipf(1.05) per table;
     mean pooling with per-sample weights N(1, 0.1); dense fp32 grad output.
  3  T=32, E=1000000 each, D cycling 64,128,256; B=16384, L ~ Poisson(20);
     Zipf(1.2) per table; sum pooling; row-wise Adagrad lr=0.01, eps=1e-8.
  4  nobag, T=1, V=131072, D=4096; 32768 token ids Zipf(1.1); bf16 grad
     N(0, 1); accumulated into an fp32 dense grad pre-filled N(0, 1).
  5  T=1, E=20000000, D=128; B=65536, L ~ U[1, 64]; Zipf(2.0); weighted sum
     pooling, weights N(1, 0.1); row-wise Adagrad lr=0.01, eps=1e-8.

Conventions: N(mu, sigma) uses sigma as the standard deviation; U[a, b] is
inclusive over integers; Zipf(alpha) is truncated to ranks 1..E with
pmf proportional to rank**-alpha, sampled by inverse CDF on the exact
normalised pmf, and row = rank - 1; Poisson(20) may give empty bags.
Random streams: numpy PCG64 seeded by SeedSequence(1000 + config).spawn(6) in
the order {lengths, indices, grad_output, per_sample_weights, weights,
momentum}.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from functools import lru_cache
from typing import Optional

import numpy as np

STREAMS = ("lengths", "indices", "grad_output", "psw", "weights", "momentum")


@dataclass
class Spec:
    """Shape and distributions of one workload (no arrays)."""
    name: str
    T: int
    E: tuple            # rows per table
    D: tuple            # embedding dim per table
    B: int              # bags per table (bag mode) / 0 for nobag without offsets
    lengths: tuple      # ("uniform", lo, hi) | ("poisson", lam) | ("fixed", n)
    index_dist: tuple   # ("uniform",) | ("zipf", alpha)
    pooling: str        # "sum" | "mean" | "none"
    weighted: bool
    grad_dtype: str     # "f32" | "bf16"
    mode: str           # "dense" | "sgd" | "rowwise_adagrad"
    accumulate: bool = False
    lr: float = 0.0
    eps: float = 0.0
    weights_std: float = 0.01      # initial weights N(0, std) (sgd/adagrad)
    dense_init_std: float = 1.0    # pre-filled dense grad N(0, std) (accumulate)
    momentum_init: str = "uniform"  # "zero" | "uniform" U[0, 1)
    nobag_tokens: int = 0           # nobag: number of token ids
    seed: int = 1000
    thr: int = 256                  # max_segment_length_per_warp used with it


CONFIGS = {
    1: Spec("c1_sgd_T1_E1000_D16", 1, (1000,), (16,), 64, ("uniform", 0, 8), ("uniform",),
            "sum", False, "f32", "sgd", lr=0.01, weights_std=0.01, seed=1001),
    2: Spec("c2_dense_T8_E100k_D128_mean_psw", 8, (100000,) * 8, (128,) * 8, 2048,
            ("uniform", 1, 32), ("zipf", 1.05), "mean", True, "f32", "dense", seed=1002),
    3: Spec("c3_adagrad_T32_E1M_Dmix_poisson20", 32, (1000000,) * 32,
            tuple((64, 128, 256)[t % 3] for t in range(32)), 16384, ("poisson", 20.0),
            ("zipf", 1.2), "sum", False, "f32", "rowwise_adagrad", lr=0.01, eps=1e-8,
            seed=1003),
    4: Spec("c4_nobag_V128k_D4096_bf16_accumulate", 1, (131072,), (4096,), 0, ("fixed", 1),
            ("zipf", 1.1), "none", False, "bf16", "dense", accumulate=True, nobag_tokens=32768,
            seed=1004),
    5: Spec("c5_adagrad_E20M_D128_zipf2_weighted", 1, (20000000,), (128,), 65536,
            ("uniform", 1, 64), ("zipf", 2.0), "sum", True, "f32", "rowwise_adagrad",
            lr=0.01, eps=1e-8, seed=1005),
}


def spec(cfg: int, **overrides) -> Spec:
    """The spec of a configuration, optionally with fields overridden.

    Overriding T with tuples left alone repeats the per-table pattern."""
    s = CONFIGS[cfg]
    if "T" in overrides and "E" not in overrides:
        overrides["E"] = tuple(s.E[t % len(s.E)] for t in range(overrides["T"]))
    if "T" in overrides and "D" not in overrides:
        overrides["D"] = tuple(s.D[t % len(s.D)] for t in range(overrides["T"]))
    if "E" in overrides and isinstance(overrides["E"], int):
        overrides["E"] = (overrides["E"],) * overrides.get("T", s.T)
    return replace(s, **overrides)


@dataclass
class Inputs:
    """Host arrays of one backward call."""
    spec: Spec
    T: int
    B: int
    hash_size_cumsum: np.ndarray     # int64 [T+1]
    D_offsets: np.ndarray            # int32 [T+1]
    offsets: Optional[np.ndarray]    # int64 [B*T+1] or None (nobag, T == 1)
    indices: np.ndarray              # int64 [N]
    per_sample_weights: Optional[np.ndarray]  # float32 [N] or None
    grad_output: np.ndarray          # float32, or uint16 bf16 bits
    rngs: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.indices.shape[0])

    @property
    def total_rows(self) -> int:
        return int(self.hash_size_cumsum[-1])

    @property
    def weights_offsets(self) -> np.ndarray:
        """Element offset of each table in the flat weight / dense-grad buffer."""
        E = np.diff(self.hash_size_cumsum)
        D = np.diff(self.D_offsets).astype(np.int64)
        return np.concatenate([[0], np.cumsum(E * D)]).astype(np.int64)


def rngs_for(seed: int) -> dict:
    ss = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(STREAMS, ss)}


@lru_cache(maxsize=8)
def _zipf_cdf(E: int, alpha: float) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    pmf = ranks ** (-alpha)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    return cdf


def zipf_rows(rng: np.random.Generator, E: int, alpha: float, n: int) -> np.ndarray:
    """n rows in [0, E): rank k in 1..E drawn with probability k**-alpha / H, row = k - 1."""
    cdf = _zipf_cdf(int(E), float(alpha))
    u = rng.random(n)
    rows = np.searchsorted(cdf, u, side="right")
    return np.minimum(rows, E - 1).astype(np.int64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bits."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _lengths(rng, dist, n) -> np.ndarray:
    if dist[0] == "uniform":
        return rng.integers(dist[1], dist[2] + 1, size=n, dtype=np.int64)
    if dist[0] == "poisson":
        return rng.poisson(dist[1], size=n).astype(np.int64)
    if dist[0] == "fixed":
        return np.full(n, dist[1], np.int64)
    raise ValueError(dist)


def generate(s: Spec, with_grad: bool = True) -> Inputs:
    """Draw the inputs of spec `s` (host numpy arrays)."""
    r = rngs_for(s.seed)
    T = s.T
    E = np.asarray(s.E, np.int64)
    D = np.asarray(s.D, np.int32)
    hsc = np.concatenate([[0], np.cumsum(E)]).astype(np.int64)
    doff = np.concatenate([[0], np.cumsum(D)]).astype(np.int32)
    nobag = s.pooling == "none"
    if nobag and s.B == 0:
        if T != 1:
            raise ValueError("nobag without offsets needs T == 1")
        offsets = None
        B = 0
        per_table = [s.nobag_tokens]
    else:
        B = s.B
        lens = _lengths(r["lengths"], s.lengths, B * T)
        offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        per_table = [int(offsets[(t + 1) * B] - offsets[t * B]) for t in range(T)]
    parts = []
    for t in range(T):
        if s.index_dist[0] == "uniform":
            parts.append(r["indices"].integers(0, E[t], size=per_table[t], dtype=np.int64))
        else:
            parts.append(zipf_rows(r["indices"], int(E[t]), s.index_dist[1], per_table[t]))
    indices = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    N = indices.shape[0]
    psw = None
    if s.weighted:
        psw = r["psw"].normal(1.0, 0.1, size=N).astype(np.float32)
    grad = None
    if with_grad:
        rows = N if nobag else B
        cols = int(D[0]) if nobag else int(doff[-1])
        g = r["grad_output"].standard_normal((rows, cols), dtype=np.float32)
        grad = bf16_bits(g) if s.grad_dtype == "bf16" else g
    return Inputs(s, T, B, hsc, doff, offsets, indices, psw, grad, r)


def initial_weights(inp: Inputs) -> np.ndarray:
    """Flat fp32 weights (or pre-filled dense grad) for the whole table set, drawn on the host.

    Only for sizes that fit comfortably in host memory (tests); large runs draw
    their initial buffers on the device instead."""
    s = inp.spec
    n = int(inp.weights_offsets[-1])
    std = s.dense_init_std if (s.mode == "dense") else s.weights_std
    return (inp.rngs["weights"].standard_normal(n, dtype=np.float32) * np.float32(std))


def initial_momentum(inp: Inputs) -> np.ndarray:
    s = inp.spec
    n = inp.total_rows
    if s.momentum_init == "zero":
        return np.zeros(n, np.float32)
    return inp.rngs["momentum"].random(n, dtype=np.float32)
