"""Parity criteria between the HIP path (fp32 arithmetic) and the binary64 oracle.

Tolerances (stated as 1e-5 relative for fp32 soft masks and logit gradients, 1e-2 for bf16
outputs), with "relative" made precise for each quantity:

* soft mask (fp32): per group of m, max_j |gpu_j - ref_j| <= tol * max_j |ref_j|.  Values far
  below the group's maximum carry errors relative to the maximum, not to themselves (a
  probability of 1e-30 is computed from an exponent of -69, whose rounding is relative to 69).
* masked weights: |gpu_j - ref_j| <= tol * max(soft mask of the group) * |w_j| + rounding of
  the output type (2^-24 |ref_j| for fp32, 1e-2 |ref_j| for bf16).
* logit gradient: grad_k = c y_k (d_k - s) is a difference, so its error is measured against the
  magnitude of the terms that form it: |gpu_k - ref_k| <= tol * c y_k (|d_k| + sum_i y_i |d_i|)
  plus an underflow floor.

tol = 1e-5 for tau >= 1/2.  Below that the fp32 noise itself limits agreement: the Gumbel
exponent is an fp32 number of magnitude up to ~25, whose rounding (~2^-24 * 25) is amplified by
1/tau; tol_for_tau scales the bound by 0.5/tau there.
"""
import numpy as np

TOL_FP32 = 1e-5
TOL_BF16 = 1e-2


def tol_for_tau(tau):
    return TOL_FP32 * max(1.0, 0.5 / float(tau))


def to_f64(t):
    """float64 numpy copy of a (GPU or CPU) torch tensor."""
    return t.detach().double().cpu().numpy()


def _diff(gpu, ref):
    """|gpu - ref|, taking equal infinities and NaN on both sides as agreement and a NaN on one
    side only as an infinite error."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    with np.errstate(invalid="ignore"):
        d = np.abs(gpu - ref)
    same = (gpu == ref) | (np.isnan(gpu) & np.isnan(ref))
    d[same] = 0.0
    d[np.isnan(d)] = np.inf
    return d


def _verdict(err, bound):
    """(largest err/bound, number of elements over their bound); a ratio <= 1 passes.  An exact
    match always passes; any other error passes only under a bound that is not NaN."""
    bad = (err != 0) & ~(err <= bound)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(err == 0, 0.0, err / np.maximum(bound, 1e-300))
    return float(np.nan_to_num(ratio, nan=np.inf).max(initial=0.0)), int(bad.sum())


def soft_mask_check(gpu, ref, m, tol):
    g = np.asarray(gpu, np.float64).reshape(-1, m)
    r = np.asarray(ref, np.float64).reshape(-1, m)
    return _verdict(_diff(g, r).max(1), tol * np.abs(r).max(1))


def forward_check(gpu, ref, w, soft_ref, m, tol, bf16):
    """gpu: float64 array of the GPU output; ref: oracle float64; w: float64 weights.
    Returns (largest error / allowed error, number of elements over it)."""
    gpu = np.asarray(gpu, np.float64)
    mmax = np.repeat(np.abs(soft_ref).reshape(-1, m).max(1), m).reshape(ref.shape)
    out_round = (TOL_BF16 if bf16 else 2.0**-24) * np.abs(ref)
    return _verdict(_diff(gpu, ref), tol * mmax * np.abs(w) + out_round)


def backward_check(gpu, ref, y, d, c, tol):
    """gpu, ref, y, d: [..., K] float64 (y = probabilities, d = candidate sums of G*w)."""
    gpu = np.asarray(gpu, np.float64)
    ad = np.abs(d)
    terms = c * y * (ad + (y * ad).sum(-1, keepdims=True))
    floor = c * 1e-36 * ad.max(-1, keepdims=True)  # probabilities near the fp32 underflow
    return _verdict(_diff(gpu, ref), tol * terms + floor)


def candidate_sums(w, grad, n, m, cand_matrix):
    """d[..., k] = sum over positions j kept by candidate k of grad_j * w_j (float64)."""
    a = (np.asarray(grad, np.float64) * np.asarray(w, np.float64))
    rows, cols = a.shape
    return a.reshape(rows, cols // m, m) @ cand_matrix.T


def candidate_sums_wreg_abs(w, grad, soft, lam, n, m, cand_matrix):
    """Size of the terms of the regularised candidate sums: per candidate k, the sum over kept
    positions j of |G_j w_j| + |2 lam w_j m_j w_j| (grad None: the regulariser alone).  The
    backward bound is relative to these magnitudes, as it is to |d| without the regulariser."""
    w = np.asarray(w, np.float64)
    a = np.abs(2.0 * lam * w * np.asarray(soft, np.float64) * w)
    if grad is not None:
        a = a + np.abs(np.asarray(grad, np.float64) * w)
    rows, cols = a.shape
    return a.reshape(rows, cols // m, m) @ cand_matrix.T


# --- convergence monitors -------------------------------------------------------------------

LN2 = 0.6931471805599453
H_ABS_MAX = 24.0   # |log2(-log2 u)| over the 2^23 uniform cells (u in [2^-24, 1 - 2^-24])


def perturbed_scores(L, kappa, tau, words, gumbel):
    """z = (kappa * l + g) / tau in float64, with g the oracle's Gumbel samples of `words`."""
    L = np.asarray(L, np.float64)
    g = np.asarray(gumbel(words), np.float64).reshape(L.shape)
    return (kappa * L + g) / tau


def sample_bound(L, kappa, tau):
    """Largest error of the kernel's fp32 comparison of two candidates' scores, in units of z,
    per group: the Gumbel exponent h = log2(-log2 u) is within 2^-21 + 2 ulp(h) (2 ulp <=
    2^-22 |h|) and enters as h / tau; the fp32 head and residual of z' = A l - B h round
    relative to |A l| + |B h| (2^-23 covers both roundings); two candidates, base 2 -> base e."""
    L = np.abs(np.asarray(L, np.float64))
    A = kappa * 1.4426950408889634 / tau
    B = 1.0 / tau
    per = B * (2.0**-21 + 2.0**-22 * H_ABS_MAX) + 2.0**-23 * (A * L.max(-1) + B * H_ABS_MAX)
    return 2.0 * LN2 * per


def sample_check(got, ref, z, bound):
    """Sampled candidates: equal wherever the oracle's top-two margin exceeds the bound; where
    they differ, the GPU's candidate scores within the bound of the top.  Returns the number of
    groups that differ (all of them near-ties)."""
    got = np.asarray(got).astype(np.int64)
    ref = np.asarray(ref).astype(np.int64)
    zs = np.sort(z, -1)
    margin = zs[..., -1] - zs[..., -2]
    diff = got != ref
    assert not (diff & (margin > bound)).any(), "sample differs where the oracle's choice is unique"
    zg = np.take_along_axis(z, got[..., None], -1)[..., 0]
    assert (zs[..., -1] - zg <= bound)[diff].all(), "sample is not among the near-tied top candidates"
    return int(diff.sum())


def l1_of(sample, prev, cand_bits):
    """Sum over groups of popcount(mask(sample) xor mask(prev)); prev >= K: the empty mask."""
    bits = np.asarray(cand_bits, np.int64)
    K = bits.size
    s = bits[np.asarray(sample).astype(np.int64)]
    p = np.asarray(prev).astype(np.int64)
    pb = np.where(p < K, bits[np.minimum(p, K - 1)], 0)
    x = s ^ pb
    return int(sum(((x >> j) & 1).sum() for j in range(8)))


# --- product with the packed weights --------------------------------------------------------

def spmm_check(gpu, ref, absterms, n_terms, bf16_out):
    """fp32 accumulation of n_terms exact products (bf16 x bf16) in any order errs by at most
    n_terms * 2^-24 * sum |x w| (the standard bound); a bf16 output adds its rounding, one unit
    in the last place of 8 bits (2^-8 |y|, covering results that round either side of a tie)."""
    gpu = np.asarray(gpu, np.float64)
    bound = n_terms * 2.0**-24 * np.asarray(absterms, np.float64)
    if bf16_out:
        bound = bound + 2.0**-8 * np.abs(ref)
    return _verdict(_diff(gpu, ref), bound + 1e-30)
