"""GPU parity of the HIP path against the oracle on small and ragged shapes, every supported
n:m, both weight types, and the edge cases (empty, one group per row, odd group counts, ties,
NaN logits, signed zeros).  Every call goes through the C ABI (semi_structured_sparsity_amd)."""
import math
import sys

import numpy as np
import pytest
import torch

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from parity import (TOL_FP32, backward_check, candidate_sums, forward_check, oracle_bounds,
                    soft_mask_check, to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SUPPORTED = [(n, m) for m in (4, 8) for n in range(1, m)]
# (rows, cols/m): ragged shapes that span several thread tiles and end in a partial tile
SHAPES = [(1, 1), (3, 5), (37, 23), (64, 64)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(rows, cols, n, m, wtype, seed, w_std=0.5):
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, wtype, w_std, seed)
    return w, L, G, w.to(DEV), L.to(DEV), G.to(DEV)


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


# ---------------------------------------------------------------------------------------------
# noise

@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("rows,gpr", SHAPES)
def test_noise_words_are_bit_exact(n, m, rows, gpr):
    seed, offset = 0x1234_5678_9ABC_DEF0 + n, 2**40 + 7 * m
    _say("noise", n, m, rows, gpr)
    got = _u32(S.nm_debug_noise(rows, gpr * m, n, m, seed, offset)).reshape(-1)
    want = oracle.noise_words(seed, offset, 0, got.size)
    np.testing.assert_array_equal(got, want)


def test_noise_beyond_2_31_slots():
    """A matrix with more than 2^31 candidate slots (64-bit slot and block arithmetic), on a few
    sampled slots."""
    rows, gpr, n, m = 22000, 16384, 2, 4  # 3.6e8 groups, 2.16e9 slots
    _say("noise large", rows * gpr)
    got = S.nm_debug_noise(rows, gpr * m, n, m, 99, 5).reshape(-1)
    last = rows * gpr * 6 - 1
    idx = [0, 1, 2**31 - 1, 2**31, 2**31 + 5, last]
    sample = got[torch.tensor(idx, device=DEV)].cpu().numpy().view(np.uint32)
    want = [oracle.noise_words(99, 5, i, 1)[0] for i in idx]
    np.testing.assert_array_equal(sample, want)
    del got
    torch.cuda.empty_cache()


def test_gumbel_transform_over_all_2_23_uniforms():
    """h = log2(-log2 u) for every 23-bit uniform, against the oracle's binary64 Gumbel sample
    g = -ln(-ln u) (h = -g log2(e) - log2(ln 2))."""
    j = np.arange(1 << 23, dtype=np.uint32)
    x = (j << np.uint32(9)) | (j & np.uint32(0x1FF))  # the low 9 bits must not matter
    h = S.nm_debug_gumbel_log2(torch.from_numpy(x.view(np.int32)).to(DEV)).double().cpu().numpy()
    g = oracle.gumbel(x)
    h_ref = -g / math.log(2) - math.log2(math.log(2))
    err = np.abs(h - h_ref)
    ulp = np.spacing(np.abs(h_ref).astype(np.float32)).astype(np.float64)
    _say("gumbel max abs err", err.max(), "max err/(2^-21 + 2 ulp(h))", (err / (2.0**-21 + 2 * ulp)).max())
    # -log2(u) to ~2 ulp relative, then the rounding of h itself
    assert np.all(err <= 2.0**-21 + 2 * ulp)


# ---------------------------------------------------------------------------------------------
# soft mask, forward, backward

# (kappa, tau): the annealing schedule's ends (100, 4) and (500, 0.05), points between, and two
# settings far outside it that the entry points also accept: nearly hard samples (2000, 0.002:
# the noise exponent's fp32 rounding is amplified 500 times) and nearly uniform ones (0.5, 50)
SAMPLES = [(100.0, 4.0), (100.0, 1.0), (1.0, 1.0), (0.0, 2.0), (30.0, 0.5), (5.0, 0.1), (3.0, 0.05),
           (500.0, 0.05), (2000.0, 0.002), (0.5, 50.0)]


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("kappa,tau", SAMPLES)
def test_soft_mask_matches_oracle(n, m, kappa, tau):
    rows, gpr = 37, 23
    _say("soft", n, m, kappa, tau)
    _, L, _, _, Ld, _ = _inputs(rows, gpr * m, n, m, torch.float32, 1)
    got = to_f64(S.nm_debug_soft_mask(Ld, n, m, kappa, tau, seed=11, offset=3))
    want = oracle.soft_mask(L, n, m, kappa, tau, 11, 3)
    _, _, dm = oracle_bounds(oracle, L, n, m, kappa, tau, 11, 3)
    rel, bad = soft_mask_check(got, want, m, TOL_FP32, dm)
    _say("  worst err/bound", rel)
    assert bad == 0
    # invariants hold on the GPU too: sum to n, within [0, 1]
    np.testing.assert_allclose(got.reshape(-1, m).sum(1), n, atol=1e-5 * n)
    assert got.min() >= 0.0 and got.max() <= 1.0 + 1e-6


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,gpr", SHAPES)
def test_forward_matches_oracle(n, m, wtype, rows, gpr):
    kappa, tau, seed, off = 100.0, 1.0, 5, 9
    _say("fwd", n, m, wtype, rows, gpr)
    w, L, _, wd, Ld, _ = _inputs(rows, gpr * m, n, m, wtype, 2)
    got = to_f64(S.nm_mask_forward(wd, Ld, n, m, kappa, tau, seed, off))
    want = oracle.forward(w, L, n, m, kappa, tau, seed, off)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off)
    rel, bad = forward_check(got, want, w.double().numpy(), soft, m, TOL_FP32,
                             wtype == torch.bfloat16)
    _say("  worst err/bound", rel)
    assert bad == 0


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,gpr", SHAPES)
def test_backward_matches_oracle(n, m, wtype, rows, gpr):
    kappa, tau, seed, off = 100.0, 1.0, 6, 2
    _say("bwd", n, m, wtype, rows, gpr)
    w, L, G, wd, Ld, Gd = _inputs(rows, gpr * m, n, m, wtype, 3)
    got = to_f64(S.nm_mask_backward(wd, Ld, Gd, n, m, kappa, tau, seed, off))
    want = oracle.backward(w, L, G, n, m, kappa, tau, seed, off)
    y = oracle.probs(L, n, m, kappa, tau, seed, off)
    d = candidate_sums(w.double().numpy(), G.double().numpy(), n, m, oracle.candidate_matrix(n, m))
    rel, bad = backward_check(got, want, y, d, kappa / tau, TOL_FP32)
    _say("  worst err/bound", rel)
    assert bad == 0


@pytest.mark.parametrize("kappa,tau", SAMPLES)
def test_backward_over_sample_parameters(kappa, tau):
    n, m, rows, gpr = 2, 4, 16, 64
    _say("bwd sample", kappa, tau)
    w, L, G, wd, Ld, Gd = _inputs(rows, gpr * m, n, m, torch.bfloat16, 4)
    got = to_f64(S.nm_mask_backward(wd, Ld, Gd, n, m, kappa, tau, 1, 1))
    want = oracle.backward(w, L, G, n, m, kappa, tau, 1, 1)
    y, dy, _ = oracle_bounds(oracle, L, n, m, kappa, tau, 1, 1)
    d = candidate_sums(w.double().numpy(), G.double().numpy(), n, m, oracle.candidate_matrix(n, m))
    rel, bad = backward_check(got, want, y, d, kappa / tau, TOL_FP32, dy=dy, n=n, m=m)
    _say("  worst err/bound", rel)
    assert bad == 0


def test_autograd_function_uses_the_same_kernels():
    n, m, rows, gpr = 2, 4, 8, 16
    w, L, G, wd, Ld, Gd = _inputs(rows, gpr * m, n, m, torch.bfloat16, 5)
    Lp = Ld.clone().requires_grad_(True)
    out = S.mask(wd, Lp, n, m, 100.0, 4.0, 3, 7)
    out.backward(Gd)
    assert torch.equal(out, S.nm_mask_forward(wd, Ld, n, m, 100.0, 4.0, 3, 7))
    assert torch.equal(Lp.grad, S.nm_mask_backward(wd, Ld, Gd, n, m, 100.0, 4.0, 3, 7))


def test_forward_and_backward_are_deterministic_and_fresh_per_step():
    n, m = 2, 4
    _, _, _, wd, Ld, Gd = _inputs(32, 256, n, m, torch.bfloat16, 6)
    a = S.nm_mask_forward(wd, Ld, n, m, 1.0, 1.0, 3, 0)
    b = S.nm_mask_forward(wd, Ld, n, m, 1.0, 1.0, 3, 0)
    c = S.nm_mask_forward(wd, Ld, n, m, 1.0, 1.0, 3, 1)
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_resume_is_exact_on_the_gpu(tmp_path):
    """Ten annealed steps straight equal five steps, a save and reload of the inputs, and the
    last five (the noise is a function of (seed, offset) alone), for the forward, backward and
    pack outputs, bit for bit."""
    n, m, seed, steps = 2, 4, 17, 10
    w, L, G = nm_synth.matrix_inputs(48, 512, n, m, torch.bfloat16, 0.02, 61, device=DEV)

    def run(w, L, G, s):
        f = s / (steps - 1)
        kappa, tau = 100.0 + 400.0 * f, 4.0 + (0.05 - 4.0) * f
        out = S.nm_mask_forward(w, L, n, m, kappa, tau, seed, s)
        dl = S.nm_mask_backward(w, L, G, n, m, kappa, tau, seed, s)
        v, i = S.nm_mask_harden_pack(w, L, n, m)
        return [t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) for t in (out, dl, v, i)]

    straight = [run(w, L, G, s) for s in range(steps)]
    torch.save({"w": w.cpu(), "L": L.cpu(), "G": G.cpu()}, tmp_path / "ckpt.pt")
    ck = torch.load(tmp_path / "ckpt.pt", weights_only=True)
    w2, L2, G2 = ck["w"].to(DEV), ck["L"].to(DEV), ck["G"].to(DEV)
    for s in range(steps // 2, steps):
        for a_, b_ in zip(straight[s], run(w2, L2, G2, s)):
            assert torch.equal(a_, b_), f"step {s} differs after the reload"


# ---------------------------------------------------------------------------------------------
# hard mask, pack, unpack: bit-exact

def _bits(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,gpr", SHAPES + [(5, 41), (7, 8), (3, 16), (2, 48), (9, 96)])
def test_harden_pack_unpack_are_bit_exact(n, m, wtype, rows, gpr):
    """Rows whose index bits fill whole words take the one-byte-per-thread path for 1:4 and 2:4
    (gpr a multiple of 8, resp. 16); the others take the chunked path."""
    _say("pack", n, m, wtype, rows, gpr)
    w, L, _, wd, Ld, _ = _inputs(rows, gpr * m, n, m, wtype, 7)
    w[0, :m] = -0.0
    L[0, 0, :] = 1.0                      # all tied: candidate 0
    if gpr > 1:
        L[0, 1, 0] = float("nan")         # NaN at 0: stays candidate 0
    if gpr > 2:
        L[0, 2, -1] = float("nan")        # NaN elsewhere: skipped
    wd, Ld = w.to(DEV), L.to(DEV)
    values, indices, hard = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=True)
    rv, ri, rh = oracle.pack(w, L, n, m)
    np.testing.assert_array_equal(hard.cpu().numpy(), rh)
    np.testing.assert_array_equal(indices.cpu().numpy().view(np.uint32), ri)
    np.testing.assert_array_equal(_bits(values), oracle._np(rv).view(_bits(values).dtype))
    dense = S.nm_unpack(values, indices, gpr * m, n, m)
    rd = oracle.unpack(rv, ri, gpr * m, n, m)
    np.testing.assert_array_equal(_bits(dense), rd.view(_bits(dense).dtype))
    # without the optional hard-index output the packed data is the same
    v2, i2 = S.nm_mask_harden_pack(wd, Ld, n, m)
    assert torch.equal(_bits_t(v2), _bits_t(values)) and torch.equal(i2, indices)


@pytest.mark.parametrize("n,m,gpr", [(3, 8, 3), (2, 4, 5), (2, 4, 16)])
def test_pack_unpack_beyond_the_grid_row_limit(n, m, gpr):
    """More rows than the tile grid's y dimension holds (65535): the tile kernels loop over
    rows; (2, 4, 16) takes the byte path with a flat grid over the same rows."""
    rows = 70001
    _say("pack rows", n, m, rows, gpr)
    w, L, _ = nm_synth.matrix_inputs(rows, gpr * m, n, m, torch.bfloat16, 0.5, 9)
    wd, Ld = w.to(DEV), L.to(DEV)
    values, indices, hard = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=True)
    rv, ri, rh = oracle.pack(w, L, n, m)
    np.testing.assert_array_equal(hard.cpu().numpy(), rh)
    np.testing.assert_array_equal(indices.cpu().numpy().view(np.uint32), ri)
    np.testing.assert_array_equal(_bits(values), oracle._np(rv).view(np.int16))
    dense = S.nm_unpack(values, indices, gpr * m, n, m)
    np.testing.assert_array_equal(_bits(dense), oracle.unpack(rv, ri, gpr * m, n, m).view(np.int16))


def _bits_t(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("n,m,gpr", [(2, 4, 19), (4, 8, 19), (3, 8, 19),
                                     (2, 4, 64), (1, 4, 64)])   # gpr 64: one thread per index byte
@pytest.mark.parametrize("wtype", [torch.bfloat16, torch.float32])
def test_unpack_of_malformed_metadata_matches_oracle(n, m, gpr, wtype):
    """Random index words: positions repeat within a group (the later field wins) and, for
    m = 8, fall past the group (skipped)."""
    rows = 6
    wpr = S.index_words_per_row(gpr * m, n, m)
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 2**32, size=(rows, wpr), dtype=np.uint64).astype(np.uint32)
    vals = nm_synth.normal((rows, gpr * n), 1.0, 8, wtype)
    got = S.nm_unpack(vals.to(DEV), torch.from_numpy(idx.view(np.int32)).to(DEV), gpr * m, n, m)
    want = oracle.unpack(vals, idx, gpr * m, n, m)
    np.testing.assert_array_equal(_bits(got), want.view(np.int16 if wtype == torch.bfloat16 else np.int32))


# ---------------------------------------------------------------------------------------------
# magnitude-prior initialisation of the logits

@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,gpr", SHAPES + [(5, 41), (129, 33)])
def test_prior_init_is_bit_exact(n, m, wtype, rows, gpr):
    _say("prior", n, m, wtype, rows, gpr)
    w = nm_synth.normal((rows, gpr * m), 0.02, 21, wtype)
    w[0, :m] = 0.25                                     # all tied: the first n positions
    if gpr > 1:
        w[0, m:2 * m] = torch.tensor([-0.5, 0.5] * (m // 2))   # tied magnitudes, opposite signs
    if gpr > 2:
        w[0, 2 * m:3 * m] = 0.0
        w[0, 2 * m + 1] = -0.0
    if gpr > 3:
        w[0, 3 * m + 1] = float("nan")                  # NaN never wins a comparison
    if gpr > 4:
        w[0, 4 * m] = float("nan")                      # NaN as the first free position
        w[0, 4 * m + 2] = float("inf")
    alpha = -2.75 if n == 3 else 3.0
    logits, idx = S.nm_prior_init(w.to(DEV), n, m, alpha, with_idx=True)
    rl, ri = oracle.prior_init(w, n, m, alpha=alpha)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(logits.cpu().numpy().view(np.uint32), rl.view(np.uint32))
    # without the optional index output the logits are the same
    assert torch.equal(S.nm_prior_init(w.to(DEV), n, m, alpha), logits)


def test_prior_init_overwrites_and_feeds_the_hard_mask():
    """Logits are overwritten (not accumulated); hardening the prior gives the prior's mask."""
    n, m, rows, cols = 2, 4, 64, 1024
    w = nm_synth.normal((rows, cols), 0.02, 22, torch.bfloat16).to(DEV)
    logits = torch.full((rows, cols // m, 6), 7.0, device=DEV)
    idx = torch.full((rows, cols // m), 255, dtype=torch.uint8, device=DEV)
    S.nm_prior_init(w, n, m, 3.0, with_idx=True, out=(logits, idx))
    assert set(torch.unique(logits).tolist()) == {0.0, 3.0}
    _, _, hard = S.nm_mask_harden_pack(w, logits, n, m, with_hard=True)
    assert torch.equal(hard, idx)
    # the kept values are the two largest magnitudes of each group
    values, _ = S.nm_mask_harden_pack(w, logits, n, m)
    top = w.float().abs().view(-1, m).topk(n, dim=1).values.sum(1)
    assert torch.equal(values.float().abs().view(-1, n).sum(1), top)


# ---------------------------------------------------------------------------------------------
# edge cases of the binding

def test_empty_matrices():
    for n, m in [(2, 4), (4, 8)]:
        K = S.num_candidates(n, m)
        w = torch.empty((0, 8 * m), dtype=torch.bfloat16, device=DEV)
        L = torch.empty((0, 8, K), device=DEV)
        assert S.nm_mask_forward(w, L, n, m, 1.0, 1.0, 0, 0).shape == (0, 8 * m)
        assert S.nm_mask_backward(w, L, w, n, m, 1.0, 1.0, 0, 0).shape == (0, 8, K)
        v, i = S.nm_mask_harden_pack(w, L, n, m)
        assert v.numel() == 0 and i.numel() == 0
        assert S.nm_prior_init(w, n, m, 3.0).shape == (0, 8, K)


def test_debug_copy_copies():
    src = torch.arange(3 * 4096 + 4, dtype=torch.int32, device=DEV)   # 16 bytes beyond whole blocks
    dst = torch.zeros_like(src)
    S.nm_debug_copy(src, dst)
    assert torch.equal(src, dst)


def test_misaligned_views_are_refused():
    n, m = 2, 4
    base = torch.zeros(4 * 64 + 2, dtype=torch.bfloat16, device=DEV)
    w = base[2:].view(4, 64)              # 4-byte offset
    L = torch.zeros(4, 16, 6, device=DEV)
    with pytest.raises(S.NMError) as e:
        S.nm_mask_forward(w, L, n, m, 1.0, 1.0, 0, 0)
    assert e.value.status == S.NM_EALIGN


def test_usage_training_loop_then_deployment():
    """The documented use: prior-initialised logits, a few optimizer steps through the
    autograd mask (gradient reaches the logits only), then harden+pack and the sparse product."""
    n, m = 2, 4
    w = nm_synth.normal((256, 256), 0.5, 51, torch.bfloat16, device=DEV)
    logits = S.nm_prior_init(w, n, m, 3.0).requires_grad_(True)
    start = logits.detach().clone()
    opt = torch.optim.SGD([logits], lr=0.1)
    for step in range(3):
        w_masked = S.mask(w, logits, n, m, 10.0, 1.0, 7, step)
        loss = (w_masked.float() ** 2).sum()
        loss.backward()
        assert logits.grad is not None and torch.isfinite(logits.grad).all()
        opt.step()
        opt.zero_grad()
    assert not torch.equal(logits.detach(), start)
    values, indices = S.nm_mask_harden_pack(w, logits.detach(), n, m)
    x = nm_synth.normal((256, 256), 1.0, 52, torch.bfloat16, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32)
    dense = S.nm_unpack(values, indices, 256, n, m).float()
    ref = x.float() @ dense.t().contiguous()
    assert torch.allclose(y, ref, rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("wtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,gpr", [(7, 32), (13, 64), (129, 32), (2, 96)])
def test_pack_groups_of_eight_flat_path_is_bit_exact(n, wtype, rows, gpr):
    """Groups of eight whose rows' fields fill whole words (gpr * n * 3 a multiple of 32) take
    the flat kernel: one partial block, several full blocks plus a partial one, and ragged
    waves; values, index words and hard indices bit-exact against the oracle, and the round
    trip through unpack exact."""
    m = 8
    if (gpr * n * 3) % 32:
        pytest.skip("not on the flat path")
    _say("pack flat8", n, wtype, rows, gpr)
    w, L, _, wd, Ld, _ = _inputs(rows, gpr * m, n, m, wtype, 91)
    values, indices, hard = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=True)
    rv, ri, rh = oracle.pack(w, L, n, m)
    assert np.array_equal(hard.cpu().numpy(), rh)
    assert np.array_equal(_u32(indices), ri)
    bits = values.view(torch.int16 if wtype == torch.bfloat16 else torch.int32).cpu().numpy()
    assert np.array_equal(bits, rv.view(bits.dtype))
    dense = S.nm_unpack(values, indices, gpr * m, n, m)
    want = oracle.unpack(rv, ri, gpr * m, n, m)
    got = dense.view(torch.int16 if wtype == torch.bfloat16 else torch.int32).cpu().numpy()
    assert np.array_equal(got, want.view(got.dtype))


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (2, 8), (4, 8)])
def test_bf16_output_is_the_rne_rounding_of_the_fp32_product(n, m):
    """The forward's bf16 output is, bit for bit, torch's round-to-nearest-even conversion of
    the fp32 product of the weights with the kernel's own fp32 soft mask (nm_debug_soft_mask
    with the same sample): the rounding step is the library routine's."""
    kappa, tau, seed, off = 100.0, 1.0, 9, 4
    _say("bf16 rne", n, m)
    _, _, _, wd, Ld, _ = _inputs(37, 23 * m, n, m, torch.bfloat16, 71)
    out = S.nm_mask_forward(wd, Ld, n, m, kappa, tau, seed, off)
    soft = S.nm_debug_soft_mask(Ld, n, m, kappa, tau, seed, off)
    want = (wd.float() * soft).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (2, 8), (4, 8)])
def test_hard_mask_is_the_large_kappa_limit_of_the_soft_mask(n, m):
    """Where kappa times a group's top-two logit gap exceeds the spread of the Gumbel noise
    (17.33 + 2.86) by 40, every other candidate's probability is below e^-39.8 (tau = 1), so the
    soft mask sampled on the GPU is the hard mask extracted on the GPU to 1e-6."""
    kappa, tau = 1.0e4, 1.0
    _say("kappa limit", n, m)
    _, _, _, wd, Ld, _ = _inputs(64, 32 * m, n, m, torch.float32, 72)
    soft = S.nm_debug_soft_mask(Ld, n, m, kappa, tau, 3, 5).view(64, 32, m)
    _, _, hard = S.nm_mask_harden_pack(wd, Ld, n, m, with_hard=True)
    table = torch.tensor(S.candidate_table(n, m), dtype=torch.int32, device=DEV)
    keep = ((table[hard.long()].unsqueeze(-1) >> torch.arange(m, device=DEV, dtype=torch.int32)) & 1).float()
    top2 = torch.topk(Ld, 2, dim=-1).values
    sure = kappa * (top2[..., 0] - top2[..., 1]) > 60.2
    assert float(sure.float().mean()) > 0.85  # most groups are decided
    err = (soft - keep).abs().amax(-1)
    assert float(err[sure].max()) <= 1e-6
