"""GPU parity of the backward with the weight regulariser (nm_mask_backward_wreg) against the
oracle: every supported n:m, both weight types, ragged shapes, with and without a task
gradient, over sample parameters, over drawn shapes, parameters and lambdas (hypothesis,
derandomized), at the full size of LLaMA-7B-shaped matrices, and through the autograd
function.  Every call goes through the C ABI."""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from oracle_inputs import oracle_prior
from parity import TOL_FP32, backward_check, candidate_sums_wreg_abs, oracle_bounds, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SUPPORTED = [(n, m) for m in (4, 8) for n in range(1, m)]
SHAPES = [(1, 1), (3, 5), (37, 23), (64, 64)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(got, w, L, G, n, m, kappa, tau, seed, off, lam, tol, rows=None, row_begin=0):
    """The stated tolerance, or where larger the bound derived from the fp32 evaluation: the
    regulariser's term 2 lam w_j m_j w_j carries the soft mask's own error dm_j into d."""
    want = oracle.backward_wreg(w, L, G, n, m, kappa, tau, seed, off, lam, rows=rows, row_begin=row_begin)
    y, dy, dm = oracle_bounds(oracle, L, n, m, kappa, tau, seed, off, rows=rows, row_begin=row_begin)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off, rows=rows, row_begin=row_begin)
    cand = oracle.candidate_matrix(n, m)
    d = candidate_sums_wreg_abs(w.double().numpy(), None if G is None else G.double().numpy(), soft,
                                lam, n, m, cand)
    wd = w.double().numpy()
    rws, cols = wd.shape
    dd = (2.0 * abs(lam) * wd * wd * dm).reshape(rws, cols // m, m) @ cand.T
    return backward_check(got, want, y, d, kappa / tau, tol, dy=dy, n=n, m=m, dd=dd)


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,gpr", SHAPES)
@pytest.mark.parametrize("lam,with_task", [(0.3, True), (-1.7, True), (0.8, False)])
def test_backward_wreg_matches_oracle(n, m, wtype, rows, gpr, lam, with_task):
    kappa, tau, seed, off = 100.0, 1.0, 6, 2
    _say("wreg", n, m, wtype, rows, gpr, lam, with_task)
    w, L, G = nm_synth.matrix_inputs(rows, gpr * m, n, m, wtype, 0.5, 31)
    G = G if with_task else None
    got = to_f64(S.nm_mask_backward_wreg(w.to(DEV), L.to(DEV), None if G is None else G.to(DEV),
                                         n, m, kappa, tau, seed, off, lam))
    rel, bad = _check(got, w, L, G, n, m, kappa, tau, seed, off, lam, TOL_FP32)
    _say("  worst err/bound", rel)
    assert bad == 0


@pytest.mark.parametrize("kappa,tau", [(100.0, 4.0), (1.0, 1.0), (0.0, 2.0), (30.0, 0.5), (5.0, 0.1), (3.0, 0.05),
                                       (500.0, 0.05)])
def test_backward_wreg_over_sample_parameters(kappa, tau):
    n, m, rows, gpr, lam = 2, 4, 16, 64, -0.6
    _say("wreg sample", kappa, tau)
    w, L, G = nm_synth.matrix_inputs(rows, gpr * m, n, m, torch.bfloat16, 0.5, 32)
    got = to_f64(S.nm_mask_backward_wreg(w.to(DEV), L.to(DEV), G.to(DEV), n, m, kappa, tau, 1, 1, lam))
    rel, bad = _check(got, w, L, G, n, m, kappa, tau, 1, 1, lam, TOL_FP32)
    _say("  worst err/bound", rel)
    assert bad == 0


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_lambda_zero_is_the_plain_backward(n, m):
    w, L, G = nm_synth.matrix_inputs(37, 23 * m, n, m, torch.bfloat16, 0.5, 33)
    wd, Ld, Gd = w.to(DEV), L.to(DEV), G.to(DEV)
    reg = S.nm_mask_backward_wreg(wd, Ld, Gd, n, m, 100.0, 4.0, 2, 3, 0.0)
    plain = S.nm_mask_backward(wd, Ld, Gd, n, m, 100.0, 4.0, 2, 3)
    assert torch.equal(reg, plain)  # -0.0 == +0.0: the only possible difference is a zero's sign


def test_autograd_function_with_regulariser():
    n, m, lam = 2, 4, -0.25
    w, L, G = nm_synth.matrix_inputs(8, 64, n, m, torch.bfloat16, 0.5, 34)
    wd, Ld, Gd = w.to(DEV), L.to(DEV), G.to(DEV)
    Lp = Ld.clone().requires_grad_(True)
    out = S.mask(wd, Lp, n, m, 100.0, 4.0, 3, 7, wreg=lam)
    out.backward(Gd)
    assert torch.equal(out, S.nm_mask_forward(wd, Ld, n, m, 100.0, 4.0, 3, 7))
    assert torch.equal(Lp.grad, S.nm_mask_backward_wreg(wd, Ld, Gd, n, m, 100.0, 4.0, 3, 7, lam))


@pytest.mark.parametrize("i", [0, 6])
@pytest.mark.parametrize("with_task", [True, False])
def test_backward_wreg_llama7b_matrix_sampled_rows(i, with_task):
    """Full LLaMA-7B-shaped matrices (q 4096x4096, down 4096x11008), launched as the benchmark
    launches them, against the oracle on sampled rows; zero-sum per group on the whole matrix."""
    n, m, kappa, tau, lam = 2, 4, 100.0, 4.0, -0.05
    name, rows, cols = nm_synth.LLAMA2_7B_LAYER[i]
    seed = nm_synth.input_seed(2, 0, i)
    _say("wreg llama", name, rows, cols, with_task)
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, logits="prior",
                                     prior=oracle_prior, device=DEV)
    G = G if with_task else None
    dl = S.nm_mask_backward_wreg(w, L, G, n, m, kappa, tau, seed, 0, lam)
    for r in sorted({0, 1, rows // 2, rows - 1}):
        Gr = None if G is None else G[r:r + 1].cpu()
        rel, bad = _check(dl[r:r + 1].double().cpu().numpy(), w[r:r + 1].cpu(), L[r:r + 1].cpu(), Gr,
                          n, m, kappa, tau, seed, 0, lam, TOL_FP32, rows=rows, row_begin=r)
        assert bad == 0, f"row {r}: {bad} elements out of tolerance (worst {rel})"
    # softmax gradients sum to zero per group, up to the rounding of their terms
    a = (w.float() ** 2).abs().view(-1, m).sum(1) * 2 * abs(lam)
    if G is not None:
        a = a + (G.float() * w.float()).abs().view(-1, m).sum(1)
    s = dl.view(-1, dl.shape[-1]).double().sum(1).abs()
    assert bool((s <= 1e-5 * (kappa / tau) * a.double() + 1e-30).all())


WREG = st.fixed_dictionaries({
    "rows": st.integers(1, 24),
    "gpr": st.integers(1, 48),
    "bf16": st.booleans(),
    "w_std": st.sampled_from([0.02, 0.5, 2.0]),
    "kappa": st.one_of(st.sampled_from([0.0, 100.0, 500.0]), st.floats(0.0, 2000.0)),
    "tau": st.one_of(st.sampled_from([0.05, 4.0]), st.floats(0.002, 50.0)),
    "lam": st.one_of(st.sampled_from([0.0, 1e-4, -3.0]), st.floats(-10.0, 10.0)),
    "with_task": st.booleans(),
    "seed": st.integers(0, 2**64 - 1),
    "offset": st.integers(0, 2**64 - 1),
    "data": st.integers(0, 2**31 - 1),
})


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (2, 8), (4, 8), (7, 8)])
@settings(max_examples=10, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(p=WREG)
def test_backward_wreg_properties(n, m, p):
    """Drawn shapes, weight types and scales, (kappa, tau), lambda (zero, tiny, negative), with
    and without a task gradient, over the whole 64-bit seed and offset ranges."""
    f32 = lambda x: float(np.float32(x))  # noqa: E731  the values the C ABI carries
    kappa, tau, lam = f32(p["kappa"]), f32(p["tau"]), f32(p["lam"])
    _say("wreg props", n, m, p["rows"], p["gpr"], p["bf16"], kappa, tau, lam, p["with_task"], p["seed"],
         p["offset"], p["data"])
    wtype = torch.bfloat16 if p["bf16"] else torch.float32
    w, L, G = nm_synth.matrix_inputs(p["rows"], p["gpr"] * m, n, m, wtype, p["w_std"], p["data"])
    G = G if p["with_task"] else None
    got = to_f64(S.nm_mask_backward_wreg(w.to(DEV), L.to(DEV), None if G is None else G.to(DEV), n, m, kappa, tau,
                                         p["seed"], p["offset"], lam))
    rel, bad = _check(got, w, L, G, n, m, kappa, tau, p["seed"], p["offset"], lam, TOL_FP32)
    assert bad == 0, f"{bad} over the bound, worst {rel}"
