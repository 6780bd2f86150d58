"""Parity at the full sizes of the benchmark workloads, launched exactly as bench.py launches
them (one C-ABI call per matrix and pass).  Where the oracle cannot cover a whole matrix in
seconds, it checks sampled rows (first, second, middle, last), and properties that hold at any
size are checked on the whole matrix on the GPU.

Workloads:
  1. one 256x256 fp32 weight, 2:4, kappa=100, tau=4, seed 0: everything, every element;
  2. one LLaMA-2-7B-shaped decoder layer (7 matrices, bf16, magnitude-prior logits);
  3. 32 such layers under the annealing schedule tau 4 -> 0.05, kappa 100 -> 500 over 10 steps
     (sampled layers and steps);
  4. every matrix of a Nemotron-15B-shaped model (32 layers x 6), pack/unpack round trip;
  5. a 4096x11008 bf16 weight with 1:4, 2:8 and 4:8.
"""
import sys

import numpy as np
import pytest
import torch

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from oracle_inputs import oracle_prior
import roundtrip_diag
from parity import (TOL_FP32, backward_check, candidate_sums, forward_check, oracle_bounds,
                    soft_mask_check, stated_excess)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _sample_rows(rows):
    return sorted({0, 1, rows // 2, rows - 1})


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _check_rows(w, L, G, n, m, kappa, tau, seed, offset, out_fwd, out_bwd, rows_to_check=None, chunk=256):
    """The oracle on whole row windows against the full-size GPU outputs: every row by default,
    in windows of `chunk` rows, or only `rows_to_check`.  The bound of each element is the stated
    tolerance or, where larger, the one derived from the kernel's fp32 evaluation (parity.py).
    Returns the largest error / bound of the forward and the backward."""
    rows = w.shape[0]
    bf16 = w.dtype == torch.bfloat16
    cand = oracle.candidate_matrix(n, m)
    windows = ([(r, r + 1) for r in rows_to_check] if rows_to_check is not None
               else [(r, min(rows, r + chunk)) for r in range(0, rows, chunk)])
    worst_f = worst_b = 0.0
    for r0, r1 in windows:
        wr, Lr = w[r0:r1].cpu(), L[r0:r1].cpu()
        wd = wr.double().numpy()
        ref = oracle.forward(wr, Lr, n, m, kappa, tau, seed, offset, rows=rows, row_begin=r0)
        y, dy, dm = oracle_bounds(oracle, Lr, n, m, kappa, tau, seed, offset, rows=rows, row_begin=r0)
        soft = (y @ cand).reshape(r1 - r0, -1)
        rel, bad = forward_check(out_fwd[r0:r1].double().cpu().numpy(), ref, wd, soft, m, TOL_FP32, bf16, dm)
        assert bad == 0, f"forward rows {r0}..{r1 - 1}: {bad} elements out of tolerance (worst {rel})"
        worst_f = max(worst_f, rel)
        if G is not None:
            Gr = G[r0:r1].cpu()
            refb = oracle.backward(wr, Lr, Gr, n, m, kappa, tau, seed, offset, rows=rows, row_begin=r0)
            d = candidate_sums(wd, Gr.double().numpy(), n, m, cand)
            got_b = out_bwd[r0:r1].double().cpu().numpy()
            rel, bad = backward_check(got_b, refb, y, d, kappa / tau, TOL_FP32, dy=dy, n=n, m=m)
            assert bad == 0, f"backward rows {r0}..{r1 - 1}: {bad} elements out of tolerance (worst {rel})"
            worst_b = max(worst_b, rel)
            over, over_rel = stated_excess(got_b, refb, y, d, kappa / tau, TOL_FP32)
            if over:
                _say(f"  rows {r0}..{r1 - 1}: {over} gradient(s) within the derived bound only,"
                     f" {over_rel:.2f} x the stated one")
    return worst_f, worst_b


def _poisoned_like(t):
    return roundtrip_diag.poisoned(tuple(t.shape), t.dtype, t.device)


def _fwd_bwd(w, L, G, n, m, kappa, tau, seed, offset):
    """Forward and backward into poisoned outputs (an unwritten element cannot pass)."""
    out = S.nm_mask_forward(w, L, n, m, kappa, tau, seed, offset, out=_poisoned_like(w))
    dl = S.nm_mask_backward(w, L, G, n, m, kappa, tau, seed, offset, out=_poisoned_like(L)) if G is not None else None
    return out, dl


_PREV_POINTERS = {}


def _check_pack_full(w, L, n, m, tag=""):
    """Whole matrix, bit-exact against the oracle; returns the GPU outputs.  Every output starts
    poisoned, and a failed round trip classifies itself (roundtrip_diag)."""
    global _PREV_POINTERS
    rows, cols = w.shape
    values, indices, hard = roundtrip_diag.pack_outputs(w, n, m, S.index_words_per_row(cols, n, m))
    S.nm_mask_harden_pack(w, L, n, m, with_hard=True, out=(values, indices, hard))
    dense = S.nm_unpack(values, indices, cols, n, m, out=roundtrip_diag.poisoned((rows, cols), w.dtype, w.device))
    rv, ri, rh = oracle.pack(w.cpu(), L.cpu(), n, m)
    assert np.array_equal(hard.cpu().numpy(), rh)
    assert np.array_equal(indices.cpu().numpy().view(np.uint32), ri)
    assert np.array_equal(_bits(values).cpu().numpy(), rv.view(_bits(values).cpu().numpy().dtype))
    # the copied-back dense weights against the oracle's unpack, and the selection on the GPU
    rd = oracle.unpack(rv, ri, cols, n, m)
    dense_ok = np.array_equal(_bits(dense).cpu().numpy(), rd.view(_bits(dense).cpu().numpy().dtype))
    keep = _keep_mask(hard, n, m)
    want = torch.where(keep, _bits(w), torch.zeros_like(_bits(w)))
    select_ok = torch.equal(_bits(dense), want)
    if not (dense_ok and select_ok):
        _report_unpack(tag, w, n, m, values, indices, hard, dense, rd, want)
    ptrs = {k: t.data_ptr() for k, t in (("values", values), ("indices", indices), ("dense", dense))}
    _PREV_POINTERS = ptrs
    assert dense_ok and select_ok
    return values, indices, hard, dense


def _report_unpack(tag, w, n, m, values, indices, hard, dense, rd, want):
    """Classify a failed unpack (roundtrip_diag) and repeat the pieces: a second copy of the
    output, the packed inputs against the oracle once more, and an unpack of the same packed
    inputs into a fresh poisoned buffer."""
    cols = w.shape[1]
    it = np.int16 if w.dtype == torch.bfloat16 else np.int32
    got = _bits(dense).cpu().numpy()
    ref = rd.view(it)
    again = _bits(dense).cpu().numpy()
    rechecks = {
        "dense_vs_oracle_wrong": int((got != ref).sum()),
        "dense_vs_selection_wrong": int((_bits(dense) != want).sum()),
        "second_copy_equal": bool(np.array_equal(again, got)),
    }
    roundtrip_diag.report(tag, w, values, indices, hard, dense, want, m, rechecks, _PREV_POINTERS, n=n)
    # then repeat the unpack: into a fresh poisoned buffer, and into the same buffer
    d2 = S.nm_unpack(values, indices, cols, n, m, out=roundtrip_diag.poisoned(tuple(w.shape), w.dtype, w.device))
    again2 = {"repeat_unpack_equals_oracle": bool(np.array_equal(_bits(d2).cpu().numpy(), ref)),
              "repeat_unpack_equals_first": bool(torch.equal(_bits(d2), _bits(dense)))}
    S.nm_unpack(values, indices, cols, n, m, out=dense)
    torch.cuda.synchronize()
    again2["same_buffer_unpack_equals_oracle"] = bool(np.array_equal(_bits(dense).cpu().numpy(), ref))
    _say("ROUND TRIP RECHECKS", again2)


def _keep_mask(hard, n, m):
    """bool [rows, cols]: the hard mask expanded from candidate indices (torch, on the GPU)."""
    table = torch.tensor(S.candidate_table(n, m), dtype=torch.int32, device=hard.device)
    bits = table[hard.long()]                                        # [rows, gpr]
    pos = torch.arange(m, device=hard.device, dtype=torch.int32)
    return ((bits.unsqueeze(-1) >> pos) & 1).bool().reshape(hard.shape[0], -1)


def _soft_properties(L, n, m, kappa, tau, seed, offset):
    """Whole matrix: every group's soft mask sums to n and lies in [0, 1]."""
    soft = S.nm_debug_soft_mask(L, n, m, kappa, tau, seed, offset)
    sums = soft.view(-1, m).double().sum(1)
    assert float((sums - n).abs().max()) <= 1e-5 * n
    assert float(soft.min()) >= 0.0 and float(soft.max()) <= 1.0 + 1e-6


def _grad_properties(w, G, dl, n, m, kappa, tau):
    """Whole matrix: the logit gradient of each group sums to zero up to rounding of its terms."""
    K = dl.shape[-1]
    a = (G.float() * w.float()).abs().view(-1, m).sum(1)
    s = dl.view(-1, K).double().sum(1).abs()
    assert bool((s <= 1e-5 * (kappa / tau) * a.double() + 1e-30).all())


# ---------------------------------------------------------------------------------------------

def test_config1_single_256x256_fp32_weight_every_element():
    n, m, kappa, tau, seed, off = 2, 4, 100.0, 4.0, 0, 0
    w, L, G = nm_synth.matrix_inputs(256, 256, n, m, torch.float32, 0.02, nm_synth.input_seed(1, 0, 0))
    wd, Ld, Gd = w.to(DEV), L.to(DEV), G.to(DEV)
    soft = S.nm_debug_soft_mask(Ld, n, m, kappa, tau, seed, off).double().cpu().numpy()
    ref_soft = oracle.soft_mask(L, n, m, kappa, tau, seed, off)
    rel, bad = soft_mask_check(soft, ref_soft, m, TOL_FP32)
    _say("config1 soft err/bound", rel)
    assert bad == 0
    out = S.nm_mask_forward(wd, Ld, n, m, kappa, tau, seed, off)
    rel, bad = forward_check(out.double().cpu().numpy(), oracle.forward(w, L, n, m, kappa, tau, seed, off),
                             w.double().numpy(), ref_soft, m, TOL_FP32, False)
    _say("config1 fwd err/bound", rel)
    assert bad == 0
    dl = S.nm_mask_backward(wd, Ld, Gd, n, m, kappa, tau, seed, off)
    y = oracle.probs(L, n, m, kappa, tau, seed, off)
    d = candidate_sums(w.double().numpy(), G.double().numpy(), n, m, oracle.candidate_matrix(n, m))
    rel, bad = backward_check(dl.double().cpu().numpy(), oracle.backward(w, L, G, n, m, kappa, tau, seed, off),
                              y, d, kappa / tau, TOL_FP32)
    _say("config1 bwd err/bound", rel)
    assert bad == 0
    words = S.nm_debug_noise(256, 256, n, m, seed, off).cpu().numpy().view(np.uint32).reshape(-1)
    assert np.array_equal(words, oracle.noise_words(seed, off, 0, words.size))
    _check_pack_full(wd, Ld, n, m, tag="config1")


@pytest.mark.parametrize("i", range(len(nm_synth.LLAMA2_7B_LAYER)))
def test_config2_llama7b_layer(i):
    n, m, kappa, tau = 2, 4, 100.0, 4.0
    name, rows, cols = nm_synth.LLAMA2_7B_LAYER[i]
    seed = nm_synth.input_seed(2, 0, i)
    _say("config2", name, rows, cols)
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, logits="prior",
                                     prior=oracle_prior, device=DEV)
    out, dl = _fwd_bwd(w, L, G, n, m, kappa, tau, seed, 0)
    wf, wb = _check_rows(w, L, G, n, m, kappa, tau, seed, 0, out, dl)
    _say("  every row: fwd/bwd err/bound", wf, wb)
    _soft_properties(L, n, m, kappa, tau, seed, 0)
    _grad_properties(w, G, dl, n, m, kappa, tau)
    _check_pack_full(w, L, n, m, tag=f"config2 {name}")
    # the prior's candidate is the hard mask wherever the prior logit margin (3) dominates
    prior = oracle_prior(w, n, m).to(DEV)
    _, _, hard = S.nm_mask_harden_pack(w, L, n, m, with_hard=True)
    assert float((hard.long() == prior).double().mean()) > 0.999
    # the prior-initialisation kernel over the whole matrix, every element against the oracle
    del out, dl, G
    Lp, ip = S.nm_prior_init(w, n, m, 3.0, with_idx=True)
    rl, ri = oracle.prior_init(w.cpu(), n, m, alpha=3.0)
    assert np.array_equal(ip.cpu().numpy(), ri)
    assert np.array_equal(Lp.cpu().numpy().view(np.uint32), rl.view(np.uint32))
    assert torch.equal(ip.long(), prior)


def _schedule(step, steps=10):
    """tau 4 -> 0.05 and kappa 100 -> 500, linear over steps 0 .. steps-1."""
    f = step / (steps - 1)
    return 100.0 + 400.0 * f, 4.0 + (0.05 - 4.0) * f


@pytest.mark.parametrize("layer,step", [(0, 0), (0, 9), (17, 4), (31, 9)])
def test_config3_annealed_sweep_sampled(layer, step):
    n, m = 2, 4
    kappa, tau = _schedule(step)
    for i, (name, rows, cols) in enumerate(nm_synth.LLAMA2_7B_LAYER):
        seed = nm_synth.input_seed(3, layer, i)
        _say("config3", layer, step, name)
        w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, logits="prior",
                                         prior=oracle_prior, device=DEV)
        out, dl = _fwd_bwd(w, L, G, n, m, kappa, tau, seed, step)
        # every row of the last layer's matrices at the last step (tau = 0.05), sampled rows elsewhere
        every = layer == 31 and step == 9
        wf, wb = _check_rows(w, L, G, n, m, kappa, tau, seed, step, out, dl,
                             rows_to_check=None if every else _sample_rows(rows))
        _say("  ", "every row" if every else "sampled rows", "fwd/bwd err/bound", wf, wb)
        _grad_properties(w, G, dl, n, m, kappa, tau)
        if step == 9:
            _check_pack_full(w, L, n, m, tag=f"config3 layer {layer} step {step} {name}")
        del w, L, G, out, dl
    torch.cuda.empty_cache()


def test_config4_nemotron15b_every_matrix_round_trip():
    """Every matrix of the Nemotron-shaped model: the hard mask is the first argmax of the
    logits (torch.argmax, which returns the first maximal index), and unpack(pack) keeps exactly
    the selected weights with +0.0 elsewhere, from poisoned outputs; the oracle checks the packed
    values, index words and hard indices of 16 rows of every matrix (the first, the last and 14
    drawn from a generator seeded by the layer and matrix)."""
    global _PREV_POINTERS
    n, m = 2, 4
    total = 0
    for layer in range(nm_synth.LAYERS):
        for i, (name, rows, cols) in enumerate(nm_synth.NEMOTRON_15B_LAYER):
            seed = nm_synth.input_seed(4, layer, i)
            w, L, _ = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.015, seed,
                                             with_grad=False, device=DEV)
            values, indices, hard = roundtrip_diag.pack_outputs(w, n, m, S.index_words_per_row(cols, n, m))
            S.nm_mask_harden_pack(w, L, n, m, with_hard=True, out=(values, indices, hard))
            dense = S.nm_unpack(values, indices, cols, n, m,
                                out=roundtrip_diag.poisoned((rows, cols), w.dtype, w.device))
            hard_ok = torch.equal(hard.long(), torch.argmax(L, dim=-1))
            keep = _keep_mask(hard, n, m)
            want = torch.where(keep, _bits(w), torch.zeros_like(_bits(w)))
            trip_ok = torch.equal(_bits(dense), want)
            if not (hard_ok and trip_ok):
                d2 = S.nm_unpack(values, indices, cols, n, m,
                                 out=roundtrip_diag.poisoned((rows, cols), w.dtype, w.device))
                v2, i2, h2 = roundtrip_diag.pack_outputs(w, n, m, S.index_words_per_row(cols, n, m))
                S.nm_mask_harden_pack(w, L, n, m, with_hard=True, out=(v2, i2, h2))
                rechecks = {"layer": layer, "matrix": name,
                            "hard_wrong": int((hard.long() != torch.argmax(L, dim=-1)).sum()),
                            "repeat_pack_values_equal": bool(torch.equal(_bits(v2), _bits(values))),
                            "repeat_pack_indices_equal": bool(torch.equal(i2, indices)),
                            "repeat_pack_hard_equal": bool(torch.equal(h2, hard)),
                            "repeat_unpack_equals_selection": bool(torch.equal(_bits(d2), want)),
                            "repeat_unpack_equals_first": bool(torch.equal(_bits(d2), _bits(dense)))}
                roundtrip_diag.report(f"config4 layer {layer} {name}", w, values, indices, hard, dense, want,
                                      m, rechecks, _PREV_POINTERS, n=n)
                S.nm_unpack(values, indices, cols, n, m, out=dense)  # again, into the same buffer
                _say("ROUND TRIP RECHECKS", {"same_buffer_unpack_equals_selection": bool(torch.equal(_bits(dense), want))})
            _PREV_POINTERS = {k: t.data_ptr() for k, t in (("values", values), ("indices", indices),
                                                            ("dense", dense))}
            assert hard_ok and trip_ok
            assert int(keep.view(-1, m).sum(1).min()) == n == int(keep.view(-1, m).sum(1).max())
            drawn = np.random.default_rng(seed).choice(np.arange(1, rows - 1), 14, replace=False)
            for r in [0, rows - 1, *sorted(int(x) for x in drawn)]:  # rows are independent
                rv, ri, rh = oracle.pack(w[r:r + 1].cpu(), L[r:r + 1].cpu(), n, m)
                assert np.array_equal(indices[r:r + 1].cpu().numpy().view(np.uint32), ri), f"{name} row {r}"
                assert np.array_equal(_bits(values[r:r + 1]).cpu().numpy(), rv.view(np.int16)), f"{name} row {r}"
                assert np.array_equal(hard[r:r + 1].cpu().numpy(), rh), f"{name} row {r}"
            total += rows * cols
            del w, L, values, indices, hard, dense, keep, want
        if layer % 8 == 7:
            _say("config4 through layer", layer)
    torch.cuda.empty_cache()
    assert total == 32 * nm_synth.layer_weights(nm_synth.NEMOTRON_15B_LAYER)


@pytest.mark.parametrize("n,m", [(1, 4), (2, 8), (4, 8)])
def test_config5_general_nm_4096x11008(n, m):
    rows, cols, kappa, tau = 4096, 11008, 100.0, 1.0
    seed = nm_synth.input_seed(5, 0, m * 10 + n)
    _say("config5", n, m)
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, seed, device=DEV)
    out, dl = _fwd_bwd(w, L, G, n, m, kappa, tau, seed, 0)
    wf, wb = _check_rows(w, L, G, n, m, kappa, tau, seed, 0, out, dl, chunk=128 if m == 8 else 256)
    _say("  every row: fwd/bwd err/bound", wf, wb)
    _soft_properties(L, n, m, kappa, tau, seed, 0)
    _grad_properties(w, G, dl, n, m, kappa, tau)
    _check_pack_full(w, L, n, m, tag=f"config5 {n}:{m}")


# ---------------------------------------------------------------------------------------------
# largest size: element offsets beyond 2^31

def test_forward_backward_pack_beyond_2_31_elements():
    """A 4096 x 786432 bf16 weight (3.2 G elements, 12.9 G bytes of logits): every 64-bit offset
    path of the forward, backward, pack and unpack, checked on sampled rows (the last one
    included) against the oracle."""
    n, m, kappa, tau = 2, 4, 100.0, 4.0
    rows, cols = 4096, 786432
    _say("beyond 2^31", rows, cols)
    w = nm_synth.normal((rows, cols), 0.02, 91, torch.bfloat16, device=DEV)
    L = nm_synth.gaussian_logits(rows, cols, n, m, 92, device=DEV)
    out = S.nm_mask_forward(w, L, n, m, kappa, tau, 5, 1)
    G = nm_synth.normal((rows, cols), 1.0, 93, torch.bfloat16, device=DEV)
    dl = S.nm_mask_backward(w, L, G, n, m, kappa, tau, 5, 1)
    torch.cuda.synchronize()
    for r in (0, 2730, rows - 1):
        wr, Lr, Gr = w[r:r + 1].cpu(), L[r:r + 1].cpu(), G[r:r + 1].cpu()
        ref = oracle.forward(wr, Lr, n, m, kappa, tau, 5, 1, rows=rows, row_begin=r)
        soft = oracle.soft_mask(Lr, n, m, kappa, tau, 5, 1, rows=rows, row_begin=r)
        _, bad = forward_check(out[r:r + 1].double().cpu().numpy(), ref, wr.double().numpy(), soft, m,
                               TOL_FP32, True)
        assert bad == 0, f"forward row {r}"
        refb = oracle.backward(wr, Lr, Gr, n, m, kappa, tau, 5, 1, rows=rows, row_begin=r)
        y = oracle.probs(Lr, n, m, kappa, tau, 5, 1, rows=rows, row_begin=r)
        d = candidate_sums(wr.double().numpy(), Gr.double().numpy(), n, m, oracle.candidate_matrix(n, m))
        _, bad = backward_check(dl[r:r + 1].double().cpu().numpy(), refb, y, d, kappa / tau, TOL_FP32)
        assert bad == 0, f"backward row {r}"
    del out, dl, G
    values, indices, hard = S.nm_mask_harden_pack(w, L, n, m, with_hard=True)
    dense = S.nm_unpack(values, indices, cols, n, m)
    for r in (1, 3001, rows - 1):
        rv, ri, rh = oracle.pack(w[r:r + 1].cpu(), L[r:r + 1].cpu(), n, m)  # rows are independent
        assert np.array_equal(hard[r:r + 1].cpu().numpy(), rh)
        assert np.array_equal(indices[r:r + 1].cpu().numpy().view(np.uint32), ri)
        assert np.array_equal(_bits(values[r:r + 1]).cpu().numpy(), oracle._np(rv).view(np.int16))
        rd = oracle.unpack(rv, ri, cols, n, m)
        assert np.array_equal(_bits(dense[r:r + 1]).cpu().numpy(), rd.view(np.int16))
    # the one-pass forward + pack on the same inputs: equal, bit for bit, to the two passes
    del dense
    fw, fv, fi, fh = S.nm_mask_forward_pack(w, L, n, m, kappa, tau, 5, 1, with_hard=True)
    assert torch.equal(_bits(fv), _bits(values)) and torch.equal(fi, indices) and torch.equal(fh, hard)
    del values, indices, hard, fv, fi, fh
    out = S.nm_mask_forward(w, L, n, m, kappa, tau, 5, 1)
    assert torch.equal(_bits(fw), _bits(out))


def test_pack_groups_of_eight_beyond_2_31_elements():
    """A 4096 x 524416 bf16 weight at 2:8 (2.15 G elements, 30 GB of logits) on the flat
    groups-of-eight kernels: every 64-bit offset of the pack and unpack, checked on sampled rows
    (the last one included) against the oracle, bit-exact."""
    n, m = 2, 8
    rows, cols = 4096, 524416  # cols/8 = 65552 groups per row: whole index words per row
    assert rows * cols > 2**31 and (cols // m * n * 3) % 32 == 0
    _say("flat8 beyond 2^31", rows, cols)
    w = nm_synth.normal((rows, cols), 0.02, 95, torch.bfloat16, device=DEV)
    L = nm_synth.gaussian_logits(rows, cols, n, m, 96, device=DEV)
    values, indices, hard = S.nm_mask_harden_pack(w, L, n, m, with_hard=True)
    dense = S.nm_unpack(values, indices, cols, n, m)
    torch.cuda.synchronize()
    for r in (0, 2731, rows - 1):
        rv, ri, rh = oracle.pack(w[r:r + 1].cpu(), L[r:r + 1].cpu(), n, m)
        assert np.array_equal(hard[r:r + 1].cpu().numpy(), rh), f"hard row {r}"
        assert np.array_equal(indices[r:r + 1].cpu().numpy().view(np.uint32), ri), f"indices row {r}"
        assert np.array_equal(_bits(values[r:r + 1]).cpu().numpy(), oracle._np(rv).view(np.int16)), f"values row {r}"
        rd = oracle.unpack(rv, ri, cols, n, m)
        assert np.array_equal(_bits(dense[r:r + 1]).cpu().numpy(), rd.view(np.int16)), f"dense row {r}"
    del w, L, values, indices, hard, dense
    torch.cuda.empty_cache()
