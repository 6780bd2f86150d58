"""The derived fp32 error bounds of tests/parity.py, checked on the CPU: an emulation of the
kernels' fp32 evaluation order (numpy float32, fused multiply-adds formed exactly in binary64
and rounded once) must stay within `prob_bound`, `soft_bound` and the derived backward bound of
the oracle's binary64 results, at the annealing schedule's ends and points between.  The Gumbel
exponent is perturbed by up to 0.95 of its measured hardware error bound (2^-21 + 2^-22 |h|),
with random signs, so the bound is exercised near its worst case.

The emulation is test scaffolding for the bound, not a second oracle: the parity of the HIP
kernels is always checked against the oracle itself."""
import numpy as np
import pytest

import oracle
from parity import LOG2E, LN2, TOL_FP32, backward_check, candidate_sums, oracle_bounds, soft_mask_check

f32 = np.float32


def _fma32(a, b, c):
    """fl32(a * b + c) with one rounding (the binary64 product of two floats is exact)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(f32)


def _emulate(L, words, kappa, tau, n, m, rng, h_err=0.95):
    """float32 (probabilities y, soft mask, e, 1/S-scaled values) in the kernels' order."""
    K = L.shape[-1]
    kf, tf = f32(kappa), f32(tau)
    A = f32(float(kf) * LOG2E / float(tf))
    B = f32(1.0 / float(tf))
    u = (words >> np.uint32(9)).astype(np.float64) * 2.0**-23 + 2.0**-24
    h64 = np.log2(-np.log2(u))
    dh = (2.0**-21 + 2.0**-22 * np.abs(h64)) * h_err * rng.uniform(-1, 1, h64.shape)
    h = (h64 + dh).astype(f32).reshape(L.shape)
    bh = (B * h).astype(f32)
    hi = _fma32(A, L, -bh)
    rem = (_fma32(A, L, -hi) - bh).astype(f32)
    mu = hi.max(-1, keepdims=True)
    t = ((hi - mu).astype(f32) + rem).astype(f32)
    e = np.exp2(t.astype(np.float64)).astype(f32)  # correctly rounded exp2 of the fp32 t
    cand = oracle.candidate_matrix(n, m).astype(bool)
    sj = np.zeros(L.shape[:-1] + (m,), f32)
    for j in range(m):
        acc = np.zeros(L.shape[:-1], f32)
        for k in range(K):
            if cand[k, j]:
                acc = (acc + e[..., k]).astype(f32)
        sj[..., j] = acc
    tot = np.zeros(L.shape[:-1], f32)
    for j in range(m):
        tot = (tot + sj[..., j]).astype(f32)
    inv = (1.0 / (tot * f32(1.0 / n)).astype(np.float64)).astype(f32)[..., None]
    y = (e * inv).astype(f32)
    soft = (sj * inv).astype(f32)
    return y, soft, e, inv


def _emulate_backward(L, words, w, G, kappa, tau, n, m, rng):
    _, _, e, inv = _emulate(L, words, kappa, tau, n, m, rng)
    K = L.shape[-1]
    rows, gpr, _ = L.shape
    a = (w.astype(f32) * G.astype(f32)).astype(f32).reshape(rows, gpr, m)
    cand = oracle.candidate_matrix(n, m).astype(bool)
    d = np.zeros(L.shape, f32)
    es = [np.zeros(L.shape[:-1], f32) for _ in range(4)]  # four interleaved fma chains
    for k in range(K):
        dk = np.zeros(L.shape[:-1], f32)
        for j in range(m):
            if cand[k, j]:
                dk = (dk + a[..., j]).astype(f32)
        d[..., k] = dk
        es[k % 4] = _fma32(e[..., k], dk, es[k % 4])
    tot = ((es[0] + es[1]).astype(f32) + (es[2] + es[3]).astype(f32)).astype(f32)
    s = (tot * inv[..., 0]).astype(f32)[..., None]
    C = f32(float(f32(kappa)) / float(f32(tau)))
    ci = (C * inv).astype(f32)
    return ((ci * e).astype(f32) * (d - s).astype(f32)).astype(f32)


CASES = [(2, 4, 100.0, 4.0), (2, 4, 500.0, 0.05), (2, 4, 3.0, 0.05), (2, 4, 5.0, 0.1), (2, 4, 30.0, 0.5),
         (4, 8, 500.0, 0.05), (4, 8, 3.0, 0.05), (2, 8, 1.0, 0.05), (1, 4, 277.8, 0.49)]


@pytest.mark.parametrize("n,m,kappa,tau", CASES)
def test_fp32_emulation_within_the_derived_probability_bound(n, m, kappa, tau):
    rng = np.random.default_rng(7)
    K = oracle.num_candidates(n, m)
    rows, gpr = 64, 96
    L = rng.standard_normal((rows, gpr, K)).astype(f32)
    if kappa >= 100:  # near-ties in kappa*l that the noise decides
        L = (L * f32(0.02)).astype(f32)
    seed, off = 3, 11
    y, dy, dm = oracle_bounds(oracle, L, n, m, kappa, tau, seed, off)
    words = oracle.noise_words(seed, off, 0, L.size)
    ye, se, _, _ = _emulate(L, words, kappa, tau, n, m, rng)
    err = np.abs(ye.astype(np.float64) - y)
    assert (err <= dy).all(), f"probability error {float((err / np.maximum(dy, 1e-300)).max())} x bound"
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off)
    rel, bad = soft_mask_check(se.reshape(rows, -1), soft, m, 0.0, dm)
    assert bad == 0, f"soft mask error {rel} x bound"
    # the derived bound is not vacuous: the emulation uses a sizeable part of it somewhere
    assert float((err / np.maximum(dy, 1e-300)).max()) > 1e-3


@pytest.mark.parametrize("n,m,kappa,tau", CASES)
def test_fp32_emulation_within_the_derived_backward_bound(n, m, kappa, tau):
    rng = np.random.default_rng(8)
    K = oracle.num_candidates(n, m)
    rows, gpr = 32, 64
    L = rng.standard_normal((rows, gpr, K)).astype(f32)
    if kappa >= 100:
        L = (L * f32(0.02)).astype(f32)
    w = (rng.standard_normal((rows, gpr * m)) * 0.5).astype(f32)
    G = rng.standard_normal((rows, gpr * m)).astype(f32)
    seed, off = 4, 2
    words = oracle.noise_words(seed, off, 0, L.size)
    got = _emulate_backward(L, words, w, G, kappa, tau, n, m, rng).astype(np.float64)
    want = oracle.backward(w, L, G, n, m, kappa, tau, seed, off)
    y, dy, _ = oracle_bounds(oracle, L, n, m, kappa, tau, seed, off)
    d = candidate_sums(w.astype(np.float64), G.astype(np.float64), n, m, oracle.candidate_matrix(n, m))
    rel, bad = backward_check(got, want, y, d, kappa / tau, 0.0, dy=dy, n=n, m=m)
    assert bad == 0, f"backward error {rel} x bound"


def test_stated_tolerance_is_below_the_fp32_limit_at_small_tau():
    """At tau = 0.05 the fp32 Gumbel exponent alone (2^-22 |h| relative) times 1/tau exceeds the
    stated 1e-5 relative error of the probabilities for typical |h|: the derived bound is the
    one that holds there, and it is larger than 1e-5 of the probability."""
    rng = np.random.default_rng(9)
    L = rng.standard_normal((16, 64, 6)).astype(f32) * f32(0.01)
    y, dy, _ = oracle_bounds(oracle, L, 2, 4, 3.0, 0.05, 1, 1)
    big = y > 0.1
    assert np.median(dy[big] / y[big]) > TOL_FP32
    y, dy, _ = oracle_bounds(oracle, L, 2, 4, 100.0, 4.0, 1, 1)
    assert (dy[y > 0.1] / y[y > 0.1]).max() < TOL_FP32  # at tau = 4 the stated bound is the larger
    assert LN2 > 0
