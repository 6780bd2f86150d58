"""GPU property tests: for every N:M pattern hypothesis draws the shape (rows, groups per row), the
weight type and scale, the logit scale, (kappa, tau) across the annealing range and far outside it
(kappa up to 5000, tau from 0.001 to 100), and the seed and offset over their whole 64-bit ranges; every pass of the path (forward, backward, harden+pack,
unpack, the monitored forward) runs through the C ABI and is compared with the oracle:
  * forward and backward within the larger of the stated 1e-5 relative bound and the derived
    fp32 bound (tests/parity.py), as the fixed parity tests;
  * packed values, index words, hard indices and the unpacked weights bit for bit;
  * the monitored forward's sampled candidates equal the oracle's except on fp32 near-ties,
    where the choice must be among the tied ones, its L1 sum is exact for its samples and its
    max-probability sum within 1e-5;
  * the magnitude prior (tied magnitudes, NaN, infinities and signed zeros at drawn places) and
    the one-call forward + pack, bit for bit.
The draws are derandomized (a fixed sequence, no example database), so a failure reproduces by
running the test again; each example prints its parameters before its GPU calls."""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from parity import (TOL_FP32, backward_check, candidate_sums, forward_check, l1_of, oracle_bounds,
                    perturbed_scores, sample_bound, sample_check, to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SUPPORTED = [(n, m) for m in (4, 8) for n in range(1, m)]
U64 = 2**64 - 1


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f32(x):
    """The fp32 value the C ABI's nm_sample carries; the oracle gets the same value."""
    return float(np.float32(x))


WIDE = st.one_of(st.integers(0, 2**16), st.integers(2**63, U64), st.integers(0, U64))
PARAMS = st.fixed_dictionaries({
    "rows": st.integers(1, 40),
    "gpr": st.integers(1, 72),
    "bf16": st.booleans(),
    "w_std": st.sampled_from([0.02, 0.5, 2.0]),
    "l_std": st.sampled_from([0.05, 1.0, 3.0]),
    "kappa": st.one_of(st.sampled_from([0.0, 100.0, 500.0]), st.floats(0.0, 500.0), st.floats(500.0, 5000.0)),
    "tau": st.one_of(st.sampled_from([0.05, 4.0]), st.floats(0.05, 4.0), st.floats(0.001, 0.05), st.floats(4.0, 100.0)),
    "seed": WIDE,
    "offset": WIDE,
    "data": st.integers(0, 2**31 - 1),
})

SETTINGS = settings(max_examples=12, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _inputs(p, n, m):
    rows, gpr = p["rows"], p["gpr"]
    wtype = torch.bfloat16 if p["bf16"] else torch.float32
    w, _, G = nm_synth.matrix_inputs(rows, gpr * m, n, m, wtype, p["w_std"], p["data"])
    L = nm_synth.gaussian_logits(rows, gpr * m, n, m, p["data"] + 1, std=p["l_std"])
    return w, L, G


@pytest.mark.parametrize("n,m", SUPPORTED)
@SETTINGS
@given(p=PARAMS)
def test_layer_passes_match_the_oracle(n, m, p):
    rows, gpr = p["rows"], p["gpr"]
    kappa, tau, seed, off = _f32(p["kappa"]), _f32(p["tau"]), p["seed"], p["offset"]
    _say("props", n, m, rows, gpr, "bf16" if p["bf16"] else "f32", kappa, tau, seed, off, p["data"])
    w, L, G = _inputs(p, n, m)
    wd, Ld, Gd = w.to(DEV), L.to(DEV), G.to(DEV)
    cand = oracle.candidate_matrix(n, m)
    y, dy, dm = oracle_bounds(oracle, L, n, m, kappa, tau, seed, off)

    got = to_f64(S.nm_mask_forward(wd, Ld, n, m, kappa, tau, seed, off))
    want = oracle.forward(w, L, n, m, kappa, tau, seed, off)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off)
    rel, bad = forward_check(got, want, w.double().numpy(), soft, m, TOL_FP32, p["bf16"], dm)
    assert bad == 0, f"forward: {bad} over the bound, worst {rel}"

    got = to_f64(S.nm_mask_backward(wd, Ld, Gd, n, m, kappa, tau, seed, off))
    want = oracle.backward(w, L, G, n, m, kappa, tau, seed, off)
    d = candidate_sums(w.double().numpy(), G.double().numpy(), n, m, cand)
    rel, bad = backward_check(got, want, y, d, _f32(kappa) / _f32(tau), TOL_FP32, dy=dy, n=n, m=m)
    assert bad == 0, f"backward: {bad} over the bound, worst {rel}"

    values, indices, hard = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=True)
    rv, ri, rh = oracle.pack(w, L, n, m)
    bits = np.int16 if p["bf16"] else np.int32
    tbits = torch.int16 if p["bf16"] else torch.int32
    np.testing.assert_array_equal(hard.cpu().numpy(), rh)
    np.testing.assert_array_equal(indices.cpu().numpy().view(np.uint32), ri)
    np.testing.assert_array_equal(values.view(tbits).cpu().numpy(), oracle._np(rv).view(bits))
    dense = S.nm_unpack(values, indices, gpr * m, n, m)
    np.testing.assert_array_equal(dense.view(tbits).cpu().numpy(), oracle.unpack(rv, ri, gpr * m, n, m).view(bits))


@pytest.mark.parametrize("n,m", SUPPORTED)
@SETTINGS
@given(p=PARAMS)
def test_monitored_forward_matches_the_oracle(n, m, p):
    rows, gpr = p["rows"], p["gpr"]
    kappa, tau, seed, off = _f32(p["kappa"]), _f32(p["tau"]), p["seed"], p["offset"]
    _say("props monitor", n, m, rows, gpr, kappa, tau, seed, off, p["data"])
    w, L, _ = _inputs(p, n, m)
    K = S.num_candidates(n, m)
    prev = np.random.default_rng(p["data"]).integers(0, K + 1, size=(rows, gpr)).astype(np.uint8)
    out, sample, stats = S.nm_mask_forward_monitor(w.to(DEV), L.to(DEV), n, m, kappa, tau, seed, off,
                                                   prev_sample=torch.from_numpy(prev).to(DEV))
    assert torch.equal(out.view(torch.int16 if p["bf16"] else torch.int32),
                       S.nm_mask_forward(w.to(DEV), L.to(DEV), n, m, kappa, tau, seed, off)
                       .view(torch.int16 if p["bf16"] else torch.int32))
    maxp, ref_s, _ = oracle.monitor(L, n, m, kappa, tau, seed, off)
    words = oracle.noise_words(seed, off, 0, L.numel())
    z = perturbed_scores(L, kappa, tau, words, oracle.gumbel)
    got = sample.cpu().numpy()
    sample_check(got, ref_s, z, sample_bound(L, kappa, tau))  # differs only on near-ties
    st_ = stats.cpu().numpy()
    assert abs(st_[0] - float(maxp.sum())) <= TOL_FP32 * float(maxp.sum())
    assert st_[1] == l1_of(got, prev, oracle.candidate_bits(n, m))


SPMM = st.fixed_dictionaries({
    "out": st.integers(1, 160).map(lambda v: 4 * v),
    "inn": st.integers(1, 48).map(lambda v: 64 * v),
    "tokens": st.one_of(st.integers(1, 4), st.integers(5, 64), st.integers(65, 600)),
    "bf16_out": st.booleans(),
    "data": st.integers(0, 2**31 - 1),
})


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(p=SPMM)
def test_sparse_product_is_exact_on_small_integers(p):
    """The product with the packed 2:4 weights over drawn shapes (every kernel path: 1-4, 5-64
    and more tokens, ragged rows and tokens): with integer weights and activations in [-8, 8]
    every product and fp32 partial sum is exact, so the result must equal the oracle's bit for
    bit (its round-to-nearest-even bf16 value for bf16 outputs)."""
    out, inn, tokens = p["out"], p["inn"], p["tokens"]
    ytype = torch.bfloat16 if p["bf16_out"] else torch.float32
    _say("props spmm", out, inn, tokens, ytype, p["data"])
    w = nm_synth.small_integers((out, inn), 8, p["data"], device=DEV)
    L = nm_synth.gaussian_logits(out, inn, 2, 4, p["data"] + 1, device=DEV)
    values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
    x = nm_synth.small_integers((tokens, inn), 8, p["data"] + 2, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=ytype)
    ref = oracle.sparse_matmul(values.cpu(), indices.cpu().numpy().view(np.uint32), x.cpu(), 2, 4)
    want = torch.from_numpy(ref).to(torch.float32).to(ytype)
    tb = torch.int16 if p["bf16_out"] else torch.int32
    assert torch.equal(y.cpu().view(tb), want.view(tb))


PRIOR = st.fixed_dictionaries({
    "rows": st.integers(1, 40),
    "gpr": st.integers(1, 72),
    "bf16": st.booleans(),
    "ints": st.booleans(),  # small-integer weights: many tied magnitudes
    "alpha": st.one_of(st.sampled_from([0.0, 3.0, -2.75]), st.floats(-1e6, 1e6)),
    "specials": st.lists(st.tuples(st.integers(0, 2**31 - 1),
                                   st.sampled_from([float("nan"), float("inf"), float("-inf"), 0.0, -0.0])),
                         max_size=6),
    "data": st.integers(0, 2**31 - 1),
})


@pytest.mark.parametrize("n,m", SUPPORTED)
@SETTINGS
@given(p=PRIOR)
def test_prior_init_matches_the_oracle(n, m, p):
    """The magnitude prior over drawn shapes, types and alphas, with tied magnitudes (small
    integers) and NaN, infinities and signed zeros at drawn places: logits and prior indices
    bit for bit."""
    rows, gpr = p["rows"], p["gpr"]
    alpha = _f32(p["alpha"])
    _say("props prior", n, m, rows, gpr, p["bf16"], p["ints"], alpha, len(p["specials"]), p["data"])
    wtype = torch.bfloat16 if p["bf16"] else torch.float32
    if p["ints"]:
        w = nm_synth.small_integers((rows, gpr * m), 3, p["data"], dtype=wtype)
    else:
        w = nm_synth.normal((rows, gpr * m), 0.02, p["data"], wtype)
    flat = w.view(-1)
    for where, value in p["specials"]:
        flat[where % flat.numel()] = value
    logits, idx = S.nm_prior_init(w.to(DEV), n, m, alpha, with_idx=True)
    rl, ri = oracle.prior_init(w, n, m, alpha=alpha)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(logits.cpu().numpy().view(np.uint32), rl.view(np.uint32))


FWD_PACK = st.fixed_dictionaries({
    "rows": st.integers(1, 40),
    "gpr": st.one_of(st.integers(1, 8).map(lambda v: 8 * v), st.integers(1, 70)),
    "bf16": st.booleans(),
    "kappa": st.one_of(st.sampled_from([0.0, 100.0, 500.0]), st.floats(0.0, 500.0)),
    "tau": st.one_of(st.sampled_from([0.05, 4.0]), st.floats(0.05, 4.0)),
    "with_hard": st.booleans(),
    "seed": WIDE,
    "offset": WIDE,
    "data": st.integers(0, 2**31 - 1),
})


@SETTINGS
@given(p=FWD_PACK)
def test_forward_pack_equals_the_two_calls(p):
    """The one-call forward + pack at 2:4 over drawn shapes (the one-pass kernel where cols / 4
    is a multiple of 8, the two calls elsewhere): its outputs equal nm_mask_forward's and
    nm_mask_harden_pack's bit for bit, and the packed form equals the oracle's."""
    n, m, rows, gpr = 2, 4, p["rows"], p["gpr"]
    kappa, tau = _f32(p["kappa"]), _f32(p["tau"])
    _say("props fwd+pack", rows, gpr, p["bf16"], kappa, tau, p["with_hard"], p["seed"], p["offset"], p["data"])
    w, L, _ = _inputs({**p, "w_std": 0.5, "l_std": 1.0}, n, m)
    wd, Ld = w.to(DEV), L.to(DEV)
    tb = torch.int16 if p["bf16"] else torch.int32
    fused = S.nm_mask_forward_pack(wd, Ld, n, m, kappa, tau, p["seed"], p["offset"], with_hard=p["with_hard"])
    assert torch.equal(fused[0].view(tb), S.nm_mask_forward(wd, Ld, n, m, kappa, tau, p["seed"], p["offset"]).view(tb))
    sep = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=p["with_hard"])
    assert torch.equal(fused[1].view(tb), sep[0].view(tb))
    assert torch.equal(fused[2], sep[1])
    rv, ri, rh = oracle.pack(w, L, n, m)
    np.testing.assert_array_equal(fused[2].cpu().numpy().view(np.uint32), ri)
    np.testing.assert_array_equal(fused[1].view(tb).cpu().numpy(), oracle._np(rv).view(np.int16 if p["bf16"] else np.int32))
    if p["with_hard"]:
        assert torch.equal(fused[3], sep[2])
        np.testing.assert_array_equal(fused[3].cpu().numpy(), rh)
