"""Pins of the oracle's differentiable mask: soft mask, forward and backward to the logits.

MaskLLM project page, Fig. 3 caption: a Gumbel-softmax sample over the candidate masks of every
group, weighted-averaged into a soft mask, all differentiable.  Fig. 5 caption: the scaling
factor kappa regulates the randomness of sampling; too small gives near-random masks, too large
freezes them.  Abstract: frozen weights.

Pins used: invariants of a probability-weighted average of n-of-m masks, closed-form special
cases (one-kept and one-dropped candidates, infinite temperature, infinite kappa, kappa = 0),
the Gumbel-max property of Gumbel noise (a textbook result), torch's fp64 softmax and autograd
as library routines, and central finite differences of the oracle's own forward.
"""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import nm_synth
import oracle

NM = [(2, 4), (1, 4), (3, 4), (2, 8), (4, 8)]


def _inputs(rows, cols, n, m, seed, wtype=torch.float32, lstd=1.0):
    w = nm_synth.normal((rows, cols), 0.5, 3 * seed, wtype)
    L = nm_synth.gaussian_logits(rows, cols, n, m, 3 * seed + 1, std=lstd)
    G = nm_synth.normal((rows, cols), 1.0, 3 * seed + 2, wtype)
    return w, L, G


def _gumbel(n, m, rows, cols, seed, offset):
    K = math.comb(m, n)
    G = rows * cols // m
    x = oracle.noise_words(seed, offset, 0, G * K)
    return torch.from_numpy(oracle.gumbel(x)).reshape(rows, cols // m, K)


# --- soft mask -------------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("kappa,tau", [(1e2, 4.0), (3.0, 1.0), (1e2, 0.05), (0.5, 10.0)])
def test_soft_mask_is_a_weighted_average_of_candidates(n, m, kappa, tau):
    rows, cols = 8, 64
    _, L, _ = _inputs(rows, cols, n, m, 1)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed=5, offset=2)
    g = soft.reshape(rows, cols // m, m)
    np.testing.assert_allclose(g.sum(-1), n, rtol=0, atol=1e-12 * n)
    assert soft.min() >= 0.0 and soft.max() <= 1.0 + 1e-15
    # y is a probability vector and the soft mask is y times the candidate matrix
    y = oracle.probs(L, n, m, kappa, tau, seed=5, offset=2)
    np.testing.assert_allclose(y.sum(-1), 1.0, atol=1e-13)
    np.testing.assert_allclose(g, y @ oracle.candidate_matrix(n, m), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("n,m", NM)
def test_probs_match_torch_softmax(n, m):
    """Library cross-check: y = torch.softmax((kappa l + g)/tau) in fp64 with the same noise."""
    rows, cols, kappa, tau, seed, off = 4, 32, 7.0, 0.7, 11, 4
    _, L, _ = _inputs(rows, cols, n, m, 2)
    y = oracle.probs(L, n, m, kappa, tau, seed, off)
    g = _gumbel(n, m, rows, cols, seed, off)
    want = torch.softmax((kappa * L.double() + g) / tau, dim=-1).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-300)


def test_one_kept_mask_equals_probabilities():
    """1:4 candidates are single positions, so the soft mask is y itself."""
    _, L, _ = _inputs(4, 32, 1, 4, 3)
    soft = oracle.soft_mask(L, 1, 4, 2.0, 1.0, 0, 0)
    y = oracle.probs(L, 1, 4, 2.0, 1.0, 0, 0)
    np.testing.assert_array_equal(soft.reshape(y.shape), y)


def test_one_dropped_mask_is_one_minus_probability():
    """3:4 candidate k drops position 3-k, so m_j = 1 - y_{3-j}."""
    _, L, _ = _inputs(4, 32, 3, 4, 4)
    soft = oracle.soft_mask(L, 3, 4, 2.0, 1.0, 0, 0).reshape(4, 8, 4)
    y = oracle.probs(L, 3, 4, 2.0, 1.0, 0, 0)
    np.testing.assert_allclose(soft, 1.0 - y[..., ::-1], atol=1e-15)


@pytest.mark.parametrize("n,m", NM)
def test_infinite_temperature_gives_uniform_mask(n, m):
    _, L, _ = _inputs(2, 32, n, m, 5)
    soft = oracle.soft_mask(L, n, m, 1.0, 1e12, 0, 0)
    np.testing.assert_allclose(soft, n / m, atol=1e-9)


@pytest.mark.parametrize("n,m", NM)
def test_infinite_kappa_gives_the_hard_mask(n, m):
    _, L, _ = _inputs(4, 64, n, m, 6)
    soft = oracle.soft_mask(L, n, m, 1e9, 1.0, 3, 1)
    hard = oracle.harden(L, n, m)
    mat = oracle.candidate_matrix(n, m)
    np.testing.assert_array_equal(soft.reshape(4, -1, m), mat[hard])


def test_kappa_zero_ignores_the_logits():
    _, L1, _ = _inputs(4, 32, 2, 4, 7)
    _, L2, _ = _inputs(4, 32, 2, 4, 8)
    a = oracle.soft_mask(L1, 2, 4, 0.0, 1.0, 9, 9)
    b = oracle.soft_mask(L2, 2, 4, 0.0, 1.0, 9, 9)
    np.testing.assert_array_equal(a, b)


def test_shift_of_a_groups_logits_leaves_its_mask_unchanged():
    _, L, _ = _inputs(4, 32, 2, 4, 9)
    L = torch.round(L * 1024) / 1024  # so that adding multiples of 1/4 is exact in fp32
    shift = torch.arange(L.shape[0] * L.shape[1], dtype=torch.float32).reshape(4, 8, 1) * 0.25
    a = oracle.soft_mask(L, 2, 4, 3.0, 0.5, 1, 1)
    b = oracle.soft_mask(L + shift, 2, 4, 3.0, 0.5, 1, 1)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


@pytest.mark.parametrize("kappa", [1.0, 2.0])
def test_gumbel_max_frequencies_follow_softmax_of_kappa_logits(kappa):
    """Gumbel-max property: argmax_k(kappa l_k + g_k) ~ Categorical(softmax(kappa l)).  At a tiny
    temperature the sampled probabilities are one-hot at that argmax, so their counts over many
    groups with the same logits must fit softmax(kappa l)."""
    l = np.array([0.3, -0.2, 0.9, 0.0, -1.1, 0.5], np.float32)
    G = 120000
    L = np.broadcast_to(l, (1, G, 6)).copy()
    y = oracle.probs(L, 2, 4, kappa, 1e-4, seed=77, offset=1)[0]
    assert (y.max(-1) > 0.999).mean() > 0.999  # one-hot except for rare near-ties
    counts = np.bincount(y.argmax(-1), minlength=6)
    p = torch.softmax(torch.tensor(kappa * l, dtype=torch.float64), 0).numpy()
    assert scipy.stats.chisquare(counts, G * p).pvalue > 1e-4
    # and the wrong law (kappa ignored) is rejected
    p_wrong = torch.softmax(torch.tensor((kappa + 1.0) * l, dtype=torch.float64), 0).numpy()
    assert scipy.stats.chisquare(counts, G * p_wrong).pvalue < 1e-6


def test_kappa_sets_the_randomness_of_sampling():
    """Fig. 5: larger kappa -> larger max probability and smaller mask change between steps;
    tiny kappa -> the change of pure noise (two independent uniform 2:4 samples differ in
    2 positions on average); huge kappa -> no change at all."""
    rows, cols = 64, 4096
    _, L, _ = _inputs(rows, cols, 2, 4, 10)
    maxp, l1_soft, l1_hard = [], [], []
    mat = oracle.candidate_matrix(2, 4)
    for kappa in [1e-3, 0.3, 1.0, 3.0, 30.0, 1e7]:
        y0 = oracle.probs(L, 2, 4, kappa, 1.0, seed=1, offset=0)
        y1 = oracle.probs(L, 2, 4, kappa, 1.0, seed=1, offset=1)
        maxp.append(y0.max(-1).mean())
        m0, m1 = y0 @ mat, y1 @ mat
        l1_soft.append(np.abs(m0 - m1).sum(-1).mean())
        h0, h1 = mat[y0.argmax(-1)], mat[y1.argmax(-1)]
        l1_hard.append(np.abs(h0 - h1).sum(-1).mean())
    assert all(a < b for a, b in zip(maxp, maxp[1:]))
    assert all(a > b for a, b in zip(l1_soft, l1_soft[1:]))
    assert all(a > b for a, b in zip(l1_hard[:-1], l1_hard[1:-1]))
    assert abs(l1_hard[0] - 2.0) < 0.02
    assert l1_hard[-1] == 0.0


# --- forward ---------------------------------------------------------------------------------

@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_forward_multiplies_the_frozen_weights(wtype):
    w, L, _ = _inputs(4, 64, 2, 4, 11, wtype)
    out = oracle.forward(w, L, 2, 4, 1e2, 4.0, 0, 0)
    soft = oracle.soft_mask(L, 2, 4, 1e2, 4.0, 0, 0)
    np.testing.assert_array_equal(out, w.double().numpy() * soft)


# --- backward --------------------------------------------------------------------------------

def _loss(w, L, G, n, m, kappa, tau, seed, off):
    return float((oracle.forward(w, L, n, m, kappa, tau, seed, off) * G.double().numpy()).sum())


@pytest.mark.parametrize("n,m,rows,cols", [(2, 4, 2, 8), (1, 4, 2, 8), (3, 4, 2, 8),
                                           (2, 8, 1, 16), (4, 8, 1, 16)])
def test_backward_matches_central_differences(n, m, rows, cols):
    kappa, tau, seed, off = 2.0, 1.5, 3, 2
    w, L, G = _inputs(rows, cols, n, m, 12)
    grad = oracle.backward(w, L, G, n, m, kappa, tau, seed, off)
    h = 2.0**-14  # exact perturbation of fp32 logits of magnitude < 2^9
    fd = np.zeros(L.shape)
    for idx in np.ndindex(*L.shape):
        Lp, Lm = L.clone(), L.clone()
        Lp[idx] += h
        Lm[idx] -= h
        fd[idx] = (_loss(w, Lp, G, n, m, kappa, tau, seed, off)
                   - _loss(w, Lm, G, n, m, kappa, tau, seed, off)) / (2 * h)
    scale = np.abs(grad).max()
    assert scale > 0
    np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-7 * scale)


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_backward_matches_torch_autograd(n, m, wtype):
    rows, cols, kappa, tau, seed, off = 4, 32, 30.0, 2.0, 9, 1
    w, L, G = _inputs(rows, cols, n, m, 13, wtype)
    grad = oracle.backward(w, L, G, n, m, kappa, tau, seed, off)
    g = _gumbel(n, m, rows, cols, seed, off)
    Ld = L.double().requires_grad_(True)
    y = torch.softmax((kappa * Ld + g) / tau, dim=-1)
    mask = (y @ torch.from_numpy(oracle.candidate_matrix(n, m))).reshape(rows, cols)
    (w.double() * mask * G.double()).sum().backward()
    np.testing.assert_allclose(grad, Ld.grad.numpy(), rtol=1e-10,
                               atol=1e-12 * np.abs(grad).max())


@pytest.mark.parametrize("n,m", NM)
def test_backward_invariants(n, m):
    """Gradients of a softmax sum to zero per group; the map is linear in the upstream grad."""
    w, L, G = _inputs(4, 64, n, m, 14)
    grad = oracle.backward(w, L, G, n, m, 5.0, 1.0, 0, 0)
    # rounding is relative to the size of the terms: (kappa/tau) * sum_j |G_j w_j| per group
    scale = 5.0 * (G.double() * w.double()).abs().reshape(grad.shape[0], grad.shape[1], m).sum(-1)
    assert np.all(np.abs(grad.sum(-1)) <= 1e-13 * scale.numpy())
    grad2 = oracle.backward(w, L, 2 * G, n, m, 5.0, 1.0, 0, 0)
    np.testing.assert_array_equal(grad2, 2 * grad)
    zero = oracle.backward(w, L, torch.zeros_like(G), n, m, 5.0, 1.0, 0, 0)
    assert not zero.any()


# --- windows, threads, resume ----------------------------------------------------------------

@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_row_windows_and_threads_do_not_change_results(n, m):
    rows, cols = 12, 64
    w, L, G = _inputs(rows, cols, n, m, 15, torch.bfloat16)
    full = oracle.backward(w, L, G, n, m, 3.0, 0.5, 21, 4, nthreads=1)
    many = oracle.backward(w, L, G, n, m, 3.0, 0.5, 21, 4, nthreads=5)
    np.testing.assert_array_equal(full, many)
    win = oracle.backward(w[5:9], L[5:9], G[5:9], n, m, 3.0, 0.5, 21, 4, rows=rows, row_begin=5)
    np.testing.assert_array_equal(win, full[5:9])
    fw = oracle.forward(w, L, n, m, 3.0, 0.5, 21, 4)
    fwin = oracle.forward(w[7:], L[7:], n, m, 3.0, 0.5, 21, 4, rows=rows, row_begin=7)
    np.testing.assert_array_equal(fwin, fw[7:])


def test_resume_is_exact(tmp_path):
    """Counter-based noise: steps 0..9 in one go equal steps 0..4, a reload, then 5..9."""
    w, L, G = _inputs(8, 64, 2, 4, 16, torch.bfloat16)
    straight = [oracle.forward(w, L, 2, 4, 1e2, 4.0, 3, s) for s in range(10)]
    np.save(tmp_path / "logits.npy", L.numpy())
    L2 = torch.from_numpy(np.load(tmp_path / "logits.npy"))
    resumed = [oracle.forward(w, L, 2, 4, 1e2, 4.0, 3, s) for s in range(5)]
    resumed += [oracle.forward(w, L2, 2, 4, 1e2, 4.0, 3, s) for s in range(5, 10)]
    for a, b in zip(straight, resumed):
        np.testing.assert_array_equal(a, b)
    assert not np.array_equal(straight[0], straight[1])  # fresh noise per step
