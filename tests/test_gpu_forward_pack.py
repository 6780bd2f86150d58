"""GPU parity of the one-call forward + pack (nm_mask_forward_pack): its outputs are bit for bit
those of nm_mask_forward and nm_mask_harden_pack on the same inputs, and those are checked
against the oracle (the forward within its tolerance, the pack bit-exact).  Covers the one-pass
kernel (2:4, cols/4 a multiple of 8), the two-pass route of every other shape, both weight
types, ragged rows, the optional hard indices and full LLaMA-7B-shaped matrices.  Every call
goes through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from oracle_inputs import oracle_prior
from parity import TOL_FP32, forward_check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16 if t.dtype in (torch.bfloat16,) else torch.int32)


def _compare_with_separate(w, L, n, m, kappa, tau, seed, off, with_hard):
    fused = S.nm_mask_forward_pack(w, L, n, m, kappa, tau, seed, off, with_hard=with_hard)
    fwd = S.nm_mask_forward(w, L, n, m, kappa, tau, seed, off)
    sep = S.nm_mask_harden_pack(w, L, n, m, with_hard=with_hard)
    assert torch.equal(_bits(fused[0]), _bits(fwd)), "w_masked differs from nm_mask_forward"
    assert torch.equal(_bits(fused[1]), _bits(sep[0])), "values differ from nm_mask_harden_pack"
    assert torch.equal(fused[2], sep[1]), "index words differ from nm_mask_harden_pack"
    if with_hard:
        assert torch.equal(fused[3], sep[2]), "hard indices differ from nm_mask_harden_pack"
    return fused


@pytest.mark.parametrize("wtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,gpr", [(1, 8), (3, 16), (37, 24), (64, 64), (5, 5), (7, 13), (2, 1)])
@pytest.mark.parametrize("with_hard", [False, True])
def test_forward_pack_2of4_equals_the_two_passes_and_the_oracle(wtype, rows, gpr, with_hard):
    n, m, kappa, tau, seed, off = 2, 4, 100.0, 1.0, 8, 3
    _say("fwd+pack", wtype, rows, gpr, with_hard)
    w, L, _ = nm_synth.matrix_inputs(rows, gpr * m, n, m, wtype, 0.5, 81)
    wd, Ld = w.to(DEV), L.to(DEV)
    out = _compare_with_separate(wd, Ld, n, m, kappa, tau, seed, off, with_hard)
    rv, ri, rh = oracle.pack(w, L, n, m)
    assert np.array_equal(_bits(out[1]).cpu().numpy(), rv.view(_bits(out[1]).cpu().numpy().dtype))
    assert np.array_equal(out[2].cpu().numpy().view(np.uint32), ri)
    if with_hard:
        assert np.array_equal(out[3].cpu().numpy(), rh)
    ref = oracle.forward(w, L, n, m, kappa, tau, seed, off)
    soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off)
    _, bad = forward_check(out[0].double().cpu().numpy(), ref, w.double().numpy(), soft, m, TOL_FP32,
                           wtype == torch.bfloat16)
    assert bad == 0


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (2, 8), (4, 8)])
def test_forward_pack_other_shapes_take_the_two_passes(n, m):
    _say("fwd+pack two passes", n, m)
    w, L, _ = nm_synth.matrix_inputs(9, 16 * m, n, m, torch.bfloat16, 0.5, 82)
    _compare_with_separate(w.to(DEV), L.to(DEV), n, m, 30.0, 0.5, 2, 9, True)


@pytest.mark.parametrize("i", [0, 6])
def test_forward_pack_llama7b_matrices(i):
    """Full LLaMA-7B-shaped matrices (q 4096x4096 and down 4096x11008), bf16, prior logits, as
    the annealed sweep's last step uses them: equal to the two passes, the pack bit-exact against
    the oracle on the whole matrix."""
    n, m, kappa, tau = 2, 4, 500.0, 0.05
    name, rows, cols = nm_synth.LLAMA2_7B_LAYER[i]
    seed = nm_synth.input_seed(3, 5, i)
    _say("fwd+pack llama", name, rows, cols)
    w, L, _ = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, logits="prior",
                                     prior=oracle_prior, device=DEV)
    out = _compare_with_separate(w, L, n, m, kappa, tau, seed, 9, True)
    rv, ri, rh = oracle.pack(w.cpu(), L.cpu(), n, m)
    assert np.array_equal(out[3].cpu().numpy(), rh)
    assert np.array_equal(out[2].cpu().numpy().view(np.uint32), ri)
    assert np.array_equal(_bits(out[1]).cpu().numpy(), rv.view(np.int16))
