"""Pins of the oracle's convergence monitors (MaskLLM project page, Fig. 5 caption: the L1
distance between masks sampled at adjacent training steps, and the largest probability of the
mask distribution as a sign of convergence).

Pins used: closed forms of the largest probability (kappa = 0, equal logits, one raised logit),
torch's fp64 softmax as a library routine, the Gumbel-max theorem (a textbook result: the
argmax of logits plus Gumbel noise is distributed as the softmax of the logits; chi-square),
the infinite-kappa and tau-invariance limits, exact ties found in the noise stream, and brute
force (set symmetric difference of itertools candidates) for the L1 distance with its
closed-form mean for independent uniform samples.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.stats
import torch

import nm_synth
import oracle

NM = [(2, 4), (1, 4), (3, 4), (2, 8), (4, 8)]


def _logits(rows, gpr, n, m, seed, std=1.0):
    return nm_synth.gaussian_logits(rows, gpr * m, n, m, seed, std=std)


# --- largest probability of the mask distribution -------------------------------------------

@pytest.mark.parametrize("n,m", NM)
def test_max_prob_closed_forms(n, m):
    K = math.comb(m, n)
    L = _logits(3, 7, n, m, 1)
    p0, _, _ = oracle.monitor(L, n, m, 0.0, 1.0, 0, 0)
    np.testing.assert_array_equal(p0, 1.0 / K)           # kappa = 0: uniform
    flat = torch.full((2, 5, K), 0.37)
    pf, _, _ = oracle.monitor(flat, n, m, 50.0, 1.0, 0, 0)
    np.testing.assert_allclose(pf, 1.0 / K, rtol=1e-15)  # equal logits: uniform
    # one logit raised by a over the others: e^(kappa a) / (e^(kappa a) + K - 1)
    one = torch.zeros((1, 4, K))
    a, kappa = 0.75, 3.0
    for q, k in enumerate([0, K - 1, K // 2, 1]):
        one[0, q, k] = a
    p1, _, _ = oracle.monitor(one, n, m, kappa, 1.0, 0, 0)
    want = math.exp(kappa * a) / (math.exp(kappa * a) + K - 1)
    np.testing.assert_allclose(p1, want, rtol=1e-14)
    # two tied maxima far above the rest at large kappa: 1/2
    two = torch.zeros((1, 1, K))
    two[0, 0, 0] = two[0, 0, K - 1] = 5.0
    p2, _, _ = oracle.monitor(two, n, m, 40.0, 1.0, 0, 0)
    assert abs(p2[0, 0] - 0.5) < 1e-80 or abs(p2[0, 0] - 0.5) < 1e-15


@pytest.mark.parametrize("n,m", NM)
def test_max_prob_matches_torch_softmax_and_ignores_noise_and_tau(n, m):
    L = _logits(5, 9, n, m, 2, std=2.0)
    for kappa in (0.3, 1.0, 7.0):
        p, _, _ = oracle.monitor(L, n, m, kappa, 0.5, 3, 4)
        want = torch.softmax(kappa * L.double(), dim=-1).max(-1).values.numpy()
        np.testing.assert_allclose(p, want, rtol=1e-13)
        q, _, _ = oracle.monitor(L, n, m, kappa, 9.0, 11, 12)   # other tau, seed and step
        np.testing.assert_array_equal(p, q)


# --- sampled mask ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", NM)
def test_sample_follows_the_gumbel_max_theorem(n, m):
    """Every group has the same logits; the sampled candidates are distributed as
    softmax(kappa * l) (chi-square), and not as softmax(l) or softmax(-kappa * l)."""
    K = math.comb(m, n)
    kappa = 1.7
    base = torch.linspace(-1.0, 1.0, K)[torch.randperm(K, generator=torch.Generator().manual_seed(K))]
    rows, gpr = 512, 128
    L = base.expand(rows, gpr, K).contiguous()
    _, s, _ = oracle.monitor(L, n, m, kappa, 0.8, 21, 5)
    counts = np.bincount(s.reshape(-1), minlength=K)
    G = rows * gpr
    p = torch.softmax(kappa * base.double(), 0).numpy()
    assert scipy.stats.chisquare(counts, G * p).pvalue > 1e-4
    for wrong in (torch.softmax(base.double(), 0).numpy(), torch.softmax(-kappa * base.double(), 0).numpy()):
        assert scipy.stats.chisquare(counts, G * wrong).pvalue < 1e-12


@pytest.mark.parametrize("n,m", NM)
def test_sample_is_uniform_at_kappa_zero(n, m):
    K = math.comb(m, n)
    L = _logits(256, 256, n, m, 3)
    _, s, _ = oracle.monitor(L, n, m, 0.0, 1.0, 8, 1)
    counts = np.bincount(s.reshape(-1), minlength=K)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4


@pytest.mark.parametrize("n,m", NM)
def test_sample_limits(n, m):
    L = _logits(16, 32, n, m, 4)
    _, s1, _ = oracle.monitor(L, n, m, 3.0, 0.25, 9, 9)
    _, s2, _ = oracle.monitor(L, n, m, 3.0, 40.0, 9, 9)
    np.testing.assert_array_equal(s1, s2)                    # tau does not change the argmax
    _, shuge, _ = oracle.monitor(L, n, m, 1e7, 1.0, 9, 9)    # noise < 30 << 1e7 * logit gaps
    np.testing.assert_array_equal(shuge, oracle.harden(L, n, m))
    # the argmax of the oracle's Gumbel-softmax probabilities (another oracle routine)
    y = oracle.probs(L, n, m, 3.0, 0.25, 9, 9)
    np.testing.assert_array_equal(s1, y.argmax(-1))


def test_sample_exact_ties_keep_the_lower_candidate():
    """At kappa = 0 the score is the Gumbel sample alone; groups whose two largest noise words
    share their top 23 bits have exactly tied scores, and the lower candidate is sampled."""
    n, m, K = 4, 8, 70   # many candidates per group: ties at the top are frequent enough
    seed, offset, chunk = 77, 3, 1 << 20
    found = []
    for c in range(8):
        j = (oracle.noise_words(seed, offset, c * chunk * K, chunk * K) >> 9).reshape(chunk, K)
        top = j.max(1)
        for g in np.nonzero((j == top[:, None]).sum(1) >= 2)[0]:
            found.append((c * chunk + int(g), int(np.nonzero(j[g] == top[g])[0][0])))
        if len(found) >= 4:
            break
    assert len(found) >= 4
    groups = 8 * chunk
    L = torch.zeros((1, 1, K))
    for g, first in found:
        # one group per row: the window is the single row g of a [groups, m] matrix
        _, s, _ = oracle.monitor(L, n, m, 0.0, 1.0, seed, offset, rows=groups, row_begin=g)
        assert s[0, 0] == first


# --- L1 distance between sampled masks ------------------------------------------------------

@pytest.mark.parametrize("n,m", NM)
def test_l1_distance_brute_force(n, m):
    K = math.comb(m, n)
    cand = [set(c) for c in itertools.combinations(range(m), n)]
    L = _logits(6, 40, n, m, 5)
    rng = np.random.default_rng(n * 10 + m)
    prev = rng.integers(0, K, size=(6, 40)).astype(np.uint8)
    prev[0, :4] = [K, 255, K + 1, 0][:4]                    # out of range: the empty mask
    _, s, l1 = oracle.monitor(L, n, m, 2.0, 1.0, 6, 7, prev_sample=prev)
    for r in range(6):
        for q in range(40):
            mine = cand[s[r, q]]
            other = cand[prev[r, q]] if prev[r, q] < K else set()
            assert l1[r, q] == len(mine ^ other)
    _, s0, l0 = oracle.monitor(L, n, m, 2.0, 1.0, 6, 7, prev_sample=s)
    np.testing.assert_array_equal(s0, s)
    np.testing.assert_array_equal(l0, 0)                    # same step: no change


@pytest.mark.parametrize("n,m", NM)
def test_l1_distance_of_independent_uniform_samples(n, m):
    """kappa = 0: adjacent steps draw independent uniform n-subsets, whose masks differ in
    2 n (m - n) / m positions on average."""
    L = _logits(128, 256, n, m, 6)
    _, s0, _ = oracle.monitor(L, n, m, 0.0, 1.0, 13, 0)
    _, _, l1 = oracle.monitor(L, n, m, 0.0, 1.0, 13, 1, prev_sample=s0)
    mean = 2 * n * (m - n) / m
    sd = l1.std() / math.sqrt(l1.size)
    assert abs(l1.mean() - mean) < 5 * sd


def test_monitor_windows_match_the_whole_matrix():
    L = _logits(9, 16, 2, 8, 7)
    prev = np.zeros((9, 16), np.uint8)
    full = oracle.monitor(L, 2, 8, 4.0, 0.5, 1, 2, prev_sample=prev)
    win = oracle.monitor(L[2:7], 2, 8, 4.0, 0.5, 1, 2, prev_sample=prev[2:7], rows=9, row_begin=2)
    for a, b in zip(full, win):
        np.testing.assert_array_equal(a[2:7], b)
