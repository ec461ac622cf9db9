"""The seeded input generators: shapes and layouts of the five workloads, the
truncated Zipf law, bf16 rounding and reproducibility (CPU only)."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_config_shapes(cfg):
    s = synth.spec(cfg)
    inp = synth.generate(s)
    T = s.T
    assert inp.hash_size_cumsum.shape == (T + 1,) and inp.hash_size_cumsum[0] == 0
    assert np.all(np.diff(inp.hash_size_cumsum) == np.asarray(s.E))
    assert np.all(np.diff(inp.D_offsets) == np.asarray(s.D))
    if s.pooling == "none":
        assert inp.offsets is None and inp.N == s.nobag_tokens
        assert inp.grad_output.shape == (inp.N, s.D[0]) and inp.grad_output.dtype == np.uint16
    else:
        assert inp.offsets.shape == (s.B * T + 1,) and inp.offsets[0] == 0
        assert inp.offsets[-1] == inp.N and np.all(np.diff(inp.offsets) >= 0)
        lens = np.diff(inp.offsets)
        lo, hi = s.lengths[1], s.lengths[2]
        assert lens.min() >= lo and lens.max() <= hi
        assert inp.grad_output.shape == (s.B, int(inp.D_offsets[-1]))
    # every index inside its table (table-major offsets give the table of a lookup)
    if inp.offsets is not None:
        for t in range(T):
            a, b = inp.offsets[t * s.B], inp.offsets[(t + 1) * s.B]
            assert np.all((inp.indices[a:b] >= 0) & (inp.indices[a:b] < s.E[t]))
    assert (inp.per_sample_weights is not None) == s.weighted


def test_reproducible():
    a = synth.generate(synth.spec(2))
    b = synth.generate(synth.spec(2))
    assert np.array_equal(a.indices, b.indices) and np.array_equal(a.offsets, b.offsets)
    assert np.array_equal(a.grad_output, b.grad_output)
    assert np.array_equal(a.per_sample_weights, b.per_sample_weights)
    c = synth.generate(synth.spec(2, seed=7))
    assert not np.array_equal(a.indices[:1000], c.indices[:1000])


def test_zipf_matches_pmf():
    """Empirical frequencies of the first ranks against k^-a / H (5 sigma)."""
    rng = np.random.default_rng(3)
    E, a, n = 1000, 1.2, 400000
    rows = synth.zipf_rows(rng, E, a, n)
    assert rows.min() >= 0 and rows.max() < E
    pmf = np.arange(1, E + 1, dtype=np.float64) ** -a
    pmf /= pmf.sum()
    cnt = np.bincount(rows, minlength=E)
    for k in range(20):
        sd = np.sqrt(n * pmf[k] * (1 - pmf[k]))
        assert abs(cnt[k] - n * pmf[k]) < 5 * sd, k


def test_zipf_alpha2_head():
    """Zipf(2) over 20M rows puts 1/zeta(2)-ish (~0.608) of the mass on row 0."""
    rng = np.random.default_rng(5)
    rows = synth.zipf_rows(rng, 20_000_000, 2.0, 200000)
    frac = np.mean(rows == 0)
    assert abs(frac - 6 / np.pi ** 2) < 0.005


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    h = synth.bf16_bits(x)
    back = synth.bf16_to_f32(h)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]
