"""Pins of the oracle's backward with the weight regulariser.

MaskLLM project page, Table 3: weight regularisation helps mask learning.  The page gives no
formula; the oracle reads it as R = lambda * sum (w * m)^2 over the masked weights, added to the
task loss.  Pins: central finite differences of that total loss through the oracle's own
binary64 forward, torch's fp64 autograd of the composite expression (library routine), the
softmax invariant (gradients of a group sum to zero), a closed form for one-kept masks, and
exact reductions (lambda = 0 is the plain backward; scaling the task gradient and lambda
together scales the result).
"""
import math

import numpy as np
import pytest
import torch

import nm_synth
import oracle

NM = [(2, 4), (1, 4), (3, 4), (2, 8), (4, 8)]


def _inputs(rows, cols, n, m, seed, wtype=torch.float32):
    w = nm_synth.normal((rows, cols), 0.5, 3 * seed, wtype)
    L = nm_synth.gaussian_logits(rows, cols, n, m, 3 * seed + 1)
    G = nm_synth.normal((rows, cols), 1.0, 3 * seed + 2, wtype)
    return w, L, G


def _gumbel(n, m, rows, cols, seed, offset):
    K = math.comb(m, n)
    x = oracle.noise_words(seed, offset, 0, rows * cols // m * K)
    return torch.from_numpy(oracle.gumbel(x)).reshape(rows, cols // m, K)


def _loss(w, L, G, lam, n, m, kappa, tau, seed, off):
    wm = oracle.forward(w, L, n, m, kappa, tau, seed, off)
    task = 0.0 if G is None else float((wm * G.double().numpy()).sum())
    return task + lam * float((wm * wm).sum())


@pytest.mark.parametrize("n,m,rows,cols", [(2, 4, 2, 8), (1, 4, 2, 8), (3, 4, 2, 8),
                                           (2, 8, 1, 16), (4, 8, 1, 16)])
@pytest.mark.parametrize("lam,with_task", [(0.7, True), (-1.3, True), (2.0, False)])
def test_backward_wreg_matches_central_differences(n, m, rows, cols, lam, with_task):
    kappa, tau, seed, off = 2.0, 1.5, 3, 2
    w, L, G = _inputs(rows, cols, n, m, 21)
    G = G if with_task else None
    grad = oracle.backward_wreg(w, L, G, n, m, kappa, tau, seed, off, lam)
    h = 2.0**-14  # exact perturbation of fp32 logits of magnitude < 2^9
    fd = np.zeros(L.shape)
    for idx in np.ndindex(*L.shape):
        Lp, Lm = L.clone(), L.clone()
        Lp[idx] += h
        Lm[idx] -= h
        fd[idx] = (_loss(w, Lp, G, lam, n, m, kappa, tau, seed, off)
                   - _loss(w, Lm, G, lam, n, m, kappa, tau, seed, off)) / (2 * h)
    scale = np.abs(grad).max()
    assert scale > 0
    np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-7 * scale)


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_backward_wreg_matches_torch_autograd(n, m, wtype):
    rows, cols, kappa, tau, seed, off, lam = 4, 32, 30.0, 2.0, 9, 1, -0.4
    w, L, G = _inputs(rows, cols, n, m, 22, wtype)
    grad = oracle.backward_wreg(w, L, G, n, m, kappa, tau, seed, off, lam)
    g = _gumbel(n, m, rows, cols, seed, off)
    Ld = L.double().requires_grad_(True)
    y = torch.softmax((kappa * Ld + g) / tau, dim=-1)
    mask = (y @ torch.from_numpy(oracle.candidate_matrix(n, m))).reshape(rows, cols)
    wm = w.double() * mask
    ((wm * G.double()).sum() + lam * (wm * wm).sum()).backward()
    np.testing.assert_allclose(grad, Ld.grad.numpy(), rtol=1e-10, atol=1e-12 * np.abs(grad).max())


def test_backward_wreg_one_kept_closed_form():
    """1:4 keeps one position per candidate, so m = y.  With no task loss,
    dR/dy_j = 2 lambda w_j^2 y_j and the softmax chain gives
    dR/dl_k = (kappa/tau) * y_k * (2 lambda w_k^2 y_k - sum_i y_i 2 lambda w_i^2 y_i)."""
    n, m, kappa, tau, seed, off, lam = 1, 4, 3.0, 0.8, 4, 7, 0.9
    w, L, _ = _inputs(3, 16, n, m, 23)
    grad = oracle.backward_wreg(w, L, None, n, m, kappa, tau, seed, off, lam)
    y = oracle.probs(L, n, m, kappa, tau, seed, off)
    w2 = (w.double().numpy() ** 2).reshape(y.shape)
    dy = 2 * lam * w2 * y
    want = (kappa / tau) * y * (dy - (y * dy).sum(-1, keepdims=True))
    np.testing.assert_allclose(grad, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("n,m", NM)
def test_backward_wreg_reductions(n, m):
    w, L, G = _inputs(4, 64, n, m, 24)
    kappa, tau = 5.0, 1.0
    plain = oracle.backward(w, L, G, n, m, kappa, tau, 0, 0)
    # lambda = 0 is the plain backward, bit for bit
    np.testing.assert_array_equal(oracle.backward_wreg(w, L, G, n, m, kappa, tau, 0, 0, 0.0), plain)
    # doubling the task gradient and lambda doubles the result exactly (binary64 scaling by 2)
    reg = oracle.backward_wreg(w, L, G, n, m, kappa, tau, 0, 0, 0.25)
    np.testing.assert_array_equal(oracle.backward_wreg(w, L, 2 * G, n, m, kappa, tau, 0, 0, 0.5), 2 * reg)
    # a regulariser alone still gives softmax gradients: they sum to zero per group
    alone = oracle.backward_wreg(w, L, None, n, m, kappa, tau, 0, 0, 1.5)
    scale = kappa * 2 * 1.5 * (w.double() ** 2).reshape(alone.shape[0], alone.shape[1], m).sum(-1)
    assert np.all(np.abs(alone.sum(-1)) <= 1e-13 * scale.numpy())
    assert np.abs(alone).max() > 0
    # the regulariser changes the gradient: it is not silently ignored
    assert not np.array_equal(reg, plain)


def test_backward_wreg_windows_use_global_noise():
    n, m, kappa, tau, seed, off, lam = 2, 4, 10.0, 2.0, 5, 3, -0.6
    w, L, G = _inputs(6, 32, n, m, 25)
    full = oracle.backward_wreg(w, L, G, n, m, kappa, tau, seed, off, lam)
    part = oracle.backward_wreg(w[2:5], L[2:5], G[2:5], n, m, kappa, tau, seed, off, lam,
                                rows=6, row_begin=2, nthreads=2)
    np.testing.assert_array_equal(part, full[2:5])
