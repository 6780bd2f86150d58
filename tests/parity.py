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

Where the kernel's fp32 evaluation cannot reach tol = 1e-5, each element's bound is the larger
of the stated one and the bound derived from that evaluation (`prob_bound` and the `dy` / `dm`
arguments below): the error of each fp32 operation of the kernel, propagated through the softmax,
the soft mask and the backward.  That happens below tau = 1/2, where the fp32 Gumbel exponent's
own rounding (2^-22 |h| relative) is amplified by 1/tau, and, at any tau, for rare logit
gradients of 4:8 groups whose value cancels (d_k close to s, a 70-term fp32 dot product).
`stated_excess` counts the elements that pass only under the derived bound.
"""
import numpy as np

TOL_FP32 = 1e-5
TOL_BF16 = 1e-2
U24 = 2.0**-24     # unit roundoff of fp32
LOG2E = 1.4426950408889634


def prob_bound(L, kappa, tau, words, gumbel, y, n, m):
    """Bound on |kernel y_k - y_k| for every candidate slot (float64, shape of L), where y are the
    oracle's binary64 probabilities and the kernel evaluates, per group and in fp32,
        h_k = log2(-log2 u_k),  hi_k = fma(A, l_k, -fl(B h_k)),  rem_k = fma(A, l_k, -hi_k) - fl(B h_k),
        t_k = (hi_k - max_i hi_i) + rem_k,  e_k = 2^t_k,  y_k = e_k / sum e
    with A = fl(kappa log2(e) / tau), B = fl(1 / tau), kappa and tau themselves rounded to fp32.

    Error of each score difference t_k - t_k* against the candidate k* with the largest exact
    score (base 2), per term:
      A and B rounded: kappa, tau and the quotient each round once (3 u for A, 2 u for B,
        u = 2^-24), times A |l_k - l_k*| and B |h_k - h_k*|;
      the Gumbel exponent: |dh| <= 2^-21 + 2^-22 |h| (measured for every 23-bit uniform), times B,
        for k and for k*;
      fl(B h) rounds (2^-24 |B h|) and is not recovered by the residual; the residual's fma and
        subtraction add as much again: 2^-23 B |h|, for k and for k*;
      hi_k - mu and the addition of rem_k round relative to |t_k|: 2^-23 |t_k|.
    With D_k that total, ln y_k = ln2 (t_k - log2 sum 2^t) changes by at most ln2 (D_k + sum y_i D_i).
    The rest is relative to y_k: the exp2 (1 ulp), the sums over candidates and positions (at
    most K + M terms), the reciprocal and the final product: (K + M + 8) u.  Below the normal
    range of fp32 (e_k < 2^-126, with the largest e about 1) the kernel may lose the whole value:
    an absolute 2^-125 covers that.  Soft-mask entries sum N of these per position
    (`soft_bound`)."""
    L = np.asarray(L, np.float64)
    y = np.asarray(y, np.float64)
    K = L.shape[-1]
    g = np.asarray(gumbel(words), np.float64).reshape(L.shape)
    h = -g * LOG2E - np.log2(LN2)
    A, B = kappa * LOG2E / tau, 1.0 / tau
    z2 = (kappa * L + g) / tau * LOG2E
    ks = np.argmax(z2, -1)[..., None]
    at = lambda a: np.take_along_axis(a, ks, -1)  # noqa: E731
    t = z2 - at(z2)
    ah = np.abs(h)
    D = (3 * U24 * A * np.abs(L - at(L)) + 2 * U24 * B * np.abs(h - at(h))
         + B * (2.0**-20 + 2.0**-22 * (ah + at(ah))) + 2.0**-23 * B * (ah + at(ah))
         + 2.0**-23 * np.abs(t) + 2.0**-60)
    dln = LN2 * (D + (y * D).sum(-1, keepdims=True))
    return y * (np.expm1(dln) + (K + m + 8) * U24) + 2.0**-125


def soft_bound(dy, n, m, cand_matrix):
    """Bound on the soft mask m_j = sum over candidates keeping j of y_k: [rows, cols]."""
    dy = np.asarray(dy, np.float64)
    rows, gpr, K = dy.shape
    return (dy @ np.asarray(cand_matrix, np.float64)).reshape(rows, gpr * m)


def oracle_bounds(oracle, L, n, m, kappa, tau, seed, offset, rows=None, row_begin=0):
    """(y, dy, dm) for a row window [row_begin, row_begin + L.shape[0]) of a rows-row matrix: the
    oracle's probabilities, and the fp32 evaluation bounds of the probabilities and soft mask."""
    L = np.asarray(oracle._np(L), np.float32)
    wr, gpr, K = L.shape
    y = oracle.probs(L, n, m, kappa, tau, seed, offset, rows=rows, row_begin=row_begin)
    words = oracle.noise_words(seed, offset, row_begin * gpr * K, wr * gpr * K)
    dy = prob_bound(L, kappa, tau, words, oracle.gumbel, y, n, m)
    return y, dy, soft_bound(dy, n, m, oracle.candidate_matrix(n, m))


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


def soft_mask_check(gpu, ref, m, tol, dm=None):
    """Per group: the stated bound tol * max |ref|, or elementwise the derived bound dm where it
    is larger."""
    g = np.asarray(gpu, np.float64).reshape(-1, m)
    r = np.asarray(ref, np.float64).reshape(-1, m)
    bound = np.repeat(tol * np.abs(r).max(1, keepdims=True), m, 1)
    if dm is not None:
        bound = np.maximum(bound, np.asarray(dm, np.float64).reshape(-1, m))
    return _verdict(_diff(g, r), bound)


def forward_check(gpu, ref, w, soft_ref, m, tol, bf16, dm=None):
    """gpu: float64 array of the GPU output; ref: oracle float64; w: float64 weights; dm: the
    derived soft-mask bound (optional).  Returns (largest error / allowed error, number of
    elements over it)."""
    gpu = np.asarray(gpu, np.float64)
    aw = np.abs(w)
    mmax = np.repeat(np.abs(soft_ref).reshape(-1, m).max(1), m).reshape(ref.shape)
    bound = tol * mmax * aw
    if dm is not None:  # the soft mask's error times |w|, and the product's rounding
        bound = np.maximum(bound, aw * (np.asarray(dm, np.float64).reshape(ref.shape) + U24 * np.abs(soft_ref)))
    out_round = (TOL_BF16 if bf16 else U24) * np.abs(ref)
    return _verdict(_diff(gpu, ref), bound + out_round)


def stated_excess(gpu, ref, y, d, c, tol):
    """(elements over the stated backward bound alone, their largest error / stated bound)."""
    gpu = np.asarray(gpu, np.float64)
    ad = np.abs(d)
    terms = c * y * (ad + (y * ad).sum(-1, keepdims=True))
    floor = c * 1e-36 * ad.max(-1, keepdims=True)
    rel, bad = _verdict(_diff(gpu, ref), tol * terms + floor)
    return bad, rel


def backward_check(gpu, ref, y, d, c, tol, dy=None, n=None, m=None, dd=None):
    """gpu, ref, y, d: [..., K] float64 (y = probabilities, d = candidate sums of G*w, or their
    magnitudes).  With dy (prob_bound) the bound is, elementwise, the larger of the stated one
    and the derived one: for grad_k = c y_k (d_k - s), s = sum_i y_i d_i,
        c (dy_k (|d_k| + |s|) + y_k sum_i dy_i |d_i|)        the probabilities' error,
        + c y_k (dd_k + sum_i y_i dd_i)                        an error of d itself (optional),
        + e c y_k (|d_k| + sum_i y_i |d_i|)                    rounding of the sums over N kept
    products, the K-term dot product with y, c = fl(kappa / tau) from fp32 kappa and tau, and
    the last products: e = (N + K + 12) u.  Plus fp32's subnormal spacing: an absolute
    2^-147 (1 + max |d|)."""
    gpu = np.asarray(gpu, np.float64)
    ad = np.abs(d)
    sy = (y * ad).sum(-1, keepdims=True)
    terms = c * y * (ad + sy)
    bound = tol * terms
    if dy is not None:
        K = ad.shape[-1]
        derived = c * (dy * (ad + sy) + y * (dy * ad).sum(-1, keepdims=True)) + (n + K + 12) * U24 * terms
        if dd is not None:
            dd = np.asarray(dd, np.float64)
            derived = derived + c * y * (dd + (y * dd).sum(-1, keepdims=True))
        bound = np.maximum(bound, derived)
    floor = c * 1e-36 * ad.max(-1, keepdims=True)  # probabilities near the fp32 underflow
    # fp32 itself: below 2^-126 its values are multiples of 2^-149, so each product of the
    # kernel's last steps (c / S, times e_k, times d_k - s) may be off by 2^-150 absolute there,
    # scaled by the factors that follow it (at most |d_k| + |s| <= 2 max |d|); a gradient below
    # 2^-149 (a tiny kappa / tau) can only come out as 0 or 2^-149
    floor = floor + 2.0**-147 * (1.0 + ad.max(-1, keepdims=True))
    return _verdict(_diff(gpu, ref), bound + floor)


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
