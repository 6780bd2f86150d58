"""Pins of the oracle's candidate table, Philox noise and Gumbel transform.

Candidates are checked against itertools (a library enumeration), the Philox block against
rocRAND's open-source Philox4x32-10 engine (an independent implementation of the SC'11
generator), and the Gumbel transform exhaustively against scipy's Gumbel quantile function
and the distribution's closed-form moments.
"""
import itertools
import math
import subprocess

import numpy as np
import pytest
import scipy.stats

import oracle


# --- candidates ------------------------------------------------------------------------------

@pytest.mark.parametrize("m", range(1, 9))
def test_candidates_are_lexicographic_n_subsets(m):
    for n in range(1, m + 1):
        bits = oracle.candidate_bits(n, m)
        expect = [sum(1 << p for p in c) for c in itertools.combinations(range(m), n)]
        assert list(bits) == expect
        assert oracle.num_candidates(n, m) == math.comb(m, n)
        mat = oracle.candidate_matrix(n, m)
        assert (mat.sum(1) == n).all()                      # each candidate keeps n
        assert (mat.sum(0) == math.comb(m - 1, n - 1)).all()  # each position in C(m-1,n-1)


def test_candidate_table_2of4():
    # the six ways to keep two of four, in the order the logits are laid out
    pos = [[j for j in range(4) if b >> j & 1] for b in oracle.candidate_bits(2, 4)]
    assert pos == [[0, 1], [0, 2], [0, 3], [1, 2], [1, 3], [2, 3]]


@pytest.mark.parametrize("n,m", [(0, 4), (5, 4), (1, 9), (-1, 4), (1, 0)])
def test_candidates_reject_bad_sizes(n, m):
    assert oracle.num_candidates(n, m) == -1


# --- Philox ----------------------------------------------------------------------------------

def _probe(probe, rows):
    text = "".join(" ".join(f"{v:x}" for v in r) + "\n" for r in rows)
    out = subprocess.run([probe], input=text, capture_output=True, text=True, check=True).stdout
    return [[int(v, 16) for v in line.split()] for line in out.strip().splitlines()]


def test_philox_block_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(20240501)
    rows = [[0] * 6, [0xFFFFFFFF] * 6, [1, 0, 0, 0, 0, 0], [0, 0, 0, 1, 0, 0],
            [0, 0, 0, 0, 0, 1]]
    rows += rng.integers(0, 2**32, size=(3000, 6), dtype=np.uint64).tolist()
    ref = _probe(rocrand_probe, rows)
    assert len(ref) == len(rows)
    for r, want in zip(rows, ref):
        got = oracle.philox4x32(r[:4], r[4:], rounds=10)
        assert list(got) == want, r


def test_noise_word_counter_map_matches_rocrand(rocrand_probe):
    """Slot i = g*K + k reads word i&3 of the block at counter (i>>2, offset), key = seed."""
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(400):
        seed = int(rng.integers(0, 2**64, dtype=np.uint64))
        offset = int(rng.integers(0, 2**64, dtype=np.uint64))
        i = int(rng.integers(0, 2**40))  # slot indices beyond 2^34 exercise the counter's high word
        cases.append((seed, offset, i))
    cases += [(0, 0, 0), (0, 0, 3), (0, 0, 4), (2**64 - 1, 2**64 - 1, 2**36 + 5)]
    rows = []
    for seed, offset, i in cases:
        b = i >> 2
        rows.append([b & 0xFFFFFFFF, b >> 32, offset & 0xFFFFFFFF, offset >> 32,
                     seed & 0xFFFFFFFF, seed >> 32])
    ref = _probe(rocrand_probe, rows)
    for (seed, offset, i), block in zip(cases, ref):
        assert oracle.noise_words(seed, offset, i, 1)[0] == block[i & 3]


def test_noise_words_statistics():
    """Top bytes uniform (chi^2), every bit balanced, neighbouring words uncorrelated."""
    N = 1 << 20
    x = oracle.noise_words(12345, 3, 0, N)
    counts = np.bincount(x >> 24, minlength=256)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    bits = ((x[:, None] >> np.arange(32)[None, :]) & 1).mean(0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / math.sqrt(N))
    u = x.astype(np.float64)
    r = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(r) < 5 / math.sqrt(N)


def test_noise_streams_differ_by_seed_and_offset():
    a = oracle.noise_words(1, 0, 0, 4096)
    b = oracle.noise_words(2, 0, 0, 4096)
    c = oracle.noise_words(1, 1, 0, 4096)
    assert (a == b).mean() < 0.01 and (a == c).mean() < 0.01
    # contiguous ranges agree with single-slot evaluation
    assert (oracle.noise_words(1, 0, 100, 8) == a[100:108]).all()


# --- uniform and Gumbel ----------------------------------------------------------------------

def test_uniform_uses_top_23_bits_at_cell_midpoints():
    for hi in [0, 1, 2**22, 2**23 - 1]:
        for lo in [0, 1, 0xFF, 0x1FF]:
            assert oracle.uniform((hi << 9) | lo) == (hi + 0.5) / 2**23
    assert 0.0 < oracle.uniform(0) and oracle.uniform(0xFFFFFFFF) < 1.0
    # every uniform is a binary32 number: 2j+1 < 2^24
    for x in [0, 0x7FFFFE00, 0xFFFFFE00, 0xFFFFFFFF]:
        u = oracle.uniform(x)
        assert float(np.float32(u)) == u


@pytest.fixture(scope="module")
def gumbel_grid():
    j = np.arange(1 << 23, dtype=np.uint32)
    return j, oracle.gumbel(j << np.uint32(9))


def test_gumbel_is_the_inverse_cdf_exhaustively(gumbel_grid):
    """All 2^23 uniforms: g equals scipy's Gumbel(0,1) quantile of u."""
    j, g = gumbel_grid
    u = (j.astype(np.float64) + 0.5) / 2**23
    want = scipy.stats.gumbel_r.ppf(u)
    np.testing.assert_allclose(g, want, rtol=2e-15, atol=2e-15)


def test_gumbel_grid_moments_and_range(gumbel_grid):
    """Mean -> Euler-Mascheroni gamma, variance -> pi^2/6; range fixed by the end cells."""
    _, g = gumbel_grid
    assert abs(g.mean() - np.euler_gamma) < 1e-5
    assert abs(g.var() - math.pi**2 / 6) < 2e-4
    assert g.min() == pytest.approx(-math.log(24 * math.log(2)), rel=1e-9)
    assert g.max() == pytest.approx(-math.log(-math.log1p(-2.0**-24)), rel=1e-9)
    assert np.all(np.diff(g) > 0)  # strictly increasing in u


def test_gumbel_ignores_low_nine_bits():
    x = np.array([0x12345600, 0x123457FF, 0x12345680], np.uint32)
    g = oracle.gumbel(x)
    assert g[0] == g[1] == g[2]
