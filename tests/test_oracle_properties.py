"""Property tests of the oracle over randomly drawn shapes, n:m and sampling parameters
(hypothesis): the invariants the pages fix must hold for every draw, not only for the fixed
cases of the other pin files."""
import math

import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import nm_synth
import oracle

NM = st.sampled_from([(1, 4), (2, 4), (3, 4), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (6, 8), (7, 8)])
SETTINGS = settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@SETTINGS
@given(nm=NM, rows=st.integers(1, 5), gpr=st.integers(1, 9), kappa=st.floats(0.0, 300.0),
       tau=st.floats(0.05, 20.0), seed=st.integers(0, 2**64 - 1), offset=st.integers(0, 2**64 - 1),
       lseed=st.integers(0, 10**6))
def test_soft_mask_sums_to_n_and_stays_in_unit_interval(nm, rows, gpr, kappa, tau, seed, offset, lseed):
    """Fig. 3 caption: a probability-weighted average of n-of-m masks keeps n per group."""
    n, m = nm
    L = nm_synth.gaussian_logits(rows, gpr * m, n, m, lseed, std=2.0)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, offset).reshape(rows, gpr, m)
    np.testing.assert_allclose(soft.sum(-1), n, rtol=0, atol=1e-9 * n)
    assert soft.min() >= 0.0 and soft.max() <= 1.0 + 1e-12


@SETTINGS
@given(nm=NM, rows=st.integers(1, 4), gpr=st.integers(1, 40), wtype=st.sampled_from([torch.float32, torch.bfloat16]),
       seed=st.integers(0, 10**6))
def test_pack_unpack_round_trip_keeps_exactly_the_hard_mask(nm, rows, gpr, wtype, seed):
    """Compressed storage: unpack(pack(w)) = w on the hard mask's n kept positions, +0 elsewhere."""
    n, m = nm
    w, L, _ = nm_synth.matrix_inputs(rows, gpr * m, n, m, wtype, 1.0, seed, with_grad=False)
    values, indices, hard = oracle.pack(w, L, n, m)
    dense = oracle._np(oracle.unpack(values, indices, gpr * m, n, m))
    wn = oracle._np(w)
    keep = oracle.candidate_matrix(n, m)[hard.astype(np.int64)].reshape(rows, gpr * m).astype(bool)
    assert (keep.reshape(rows, gpr, m).sum(-1) == n).all()
    np.testing.assert_array_equal(dense[keep], wn[keep])
    assert (dense[~keep].view(np.uint16 if dense.dtype == np.uint16 else np.uint32) == 0).all()  # +0.0 bits
    assert indices.shape[1] == math.ceil(gpr * n * (m - 1).bit_length() / 32)


@SETTINGS
@given(nm=NM, rows=st.integers(1, 3), gpr=st.integers(1, 6), kappa=st.floats(0.1, 20.0),
       tau=st.floats(0.2, 5.0), seed=st.integers(0, 2**32), gseed=st.integers(0, 10**6))
def test_logit_gradient_sums_to_zero_per_group(nm, rows, gpr, kappa, tau, seed, gseed):
    """Softmax Jacobian: adding a constant to a group's logits changes nothing, so the gradient
    of every group sums to zero (up to rounding of its terms)."""
    n, m = nm
    w, L, G = nm_synth.matrix_inputs(rows, gpr * m, n, m, torch.float32, 1.0, gseed)
    dl = oracle.backward(w, L, G, n, m, kappa, tau, seed, 3)
    scale = (kappa / tau) * np.abs(G.double().numpy() * w.double().numpy()).reshape(rows, gpr, m).sum(-1) * n
    assert (np.abs(dl.sum(-1)) <= 1e-12 * scale + 1e-300).all()


@SETTINGS
@given(nm=NM, rows=st.integers(1, 3), gpr=st.integers(1, 12), seed=st.integers(0, 10**6),
       alpha=st.floats(-10.0, 10.0))
def test_prior_keeps_the_n_largest_magnitudes(nm, rows, gpr, seed, alpha):
    n, m = nm
    w = nm_synth.normal((rows, gpr * m), 1.0, seed, torch.bfloat16)
    logits, idx = oracle.prior_init(w, n, m, alpha=alpha)
    mags = np.abs(w.float().numpy()).reshape(rows, gpr, m)
    keep = oracle.candidate_matrix(n, m)[idx.astype(np.int64)].astype(bool)
    # every kept magnitude is at least every dropped one
    kept_min = np.where(keep, mags, np.inf).min(-1)
    drop_max = np.where(keep, -np.inf, mags).max(-1)
    assert (kept_min >= drop_max).all()
    assert (logits.sum(-1) == np.float32(alpha)).all() and (np.count_nonzero(logits, -1) <= 1).all()
