"""Host-side tests of the C ABI (no GPU): exported symbols, argument validation before any HIP
call, and the host helpers, which are compared with the oracle's independent versions."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import semi_structured_sparsity_amd as S
from semi_structured_sparsity_amd import NM_EALIGN, NM_EINVAL, NM_EUNSUPPORTED, NM_OK

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUPPORTED = [(n, m) for m in (4, 8) for n in range(1, m)]


def _declared():
    text = open(os.path.join(ROOT, "include", "nm_mask.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = S.lib()
    declared = _declared()
    assert len(declared) >= 18
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(S.EXPORTS)


def _shape(rows=4, cols=16, n=2, m=4, wtype=0):
    return ctypes.byref(S._Shape(rows, cols, n, m, wtype))


def _sample(kappa=1.0, tau=1.0):
    return ctypes.byref(S._Sample(kappa, tau, 0, 0))


FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p((1 << 20) + 4)     # misaligned


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), NM_EINVAL), (dict(cols=-4), NM_EINVAL), (dict(cols=6), NM_EINVAL),
    (dict(n=0), NM_EUNSUPPORTED), (dict(n=4), NM_EUNSUPPORTED), (dict(m=6, n=2, cols=12), NM_EUNSUPPORTED),
    (dict(m=16, n=2), NM_EUNSUPPORTED), (dict(wtype=2), NM_EUNSUPPORTED),
    (dict(rows=2**40, cols=2**40), NM_EINVAL),
])
def test_bad_shapes_are_rejected_on_the_host(kw, status):
    L = S.lib()
    sh = _shape(**kw)
    assert L.nm_mask_forward(sh, _sample(), FAKE, FAKE, FAKE, None) == status
    assert L.nm_mask_backward(sh, _sample(), FAKE, FAKE, FAKE, FAKE, None) == status
    assert L.nm_mask_backward_wreg(sh, _sample(), 0.5, FAKE, FAKE, FAKE, FAKE, None) == status
    assert L.nm_mask_harden_pack(sh, FAKE, FAKE, FAKE, FAKE, None, None) == status
    assert L.nm_mask_forward_pack(sh, _sample(), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == status
    assert L.nm_unpack(sh, FAKE, FAKE, FAKE, None) == status
    assert L.nm_debug_noise(sh, _sample(), FAKE, None) == status
    assert L.nm_debug_soft_mask(sh, _sample(), FAKE, FAKE, None) == status
    assert L.nm_prior_init(sh, 3.0, FAKE, FAKE, FAKE, None) == status
    assert L.nm_mask_forward_monitor(sh, _sample(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     1 << 40, None) == status
    assert L.nm_monitor_workspace_bytes(sh) == -1
    assert L.nm_packed_value_elems(sh) == -1 and L.nm_index_words_per_row(sh) == -1


@pytest.mark.parametrize("kappa,tau", [(-1.0, 1.0), (float("nan"), 1.0), (float("inf"), 1.0),
                                       (1.0, 0.0), (1.0, -2.0), (1.0, float("nan")),
                                       (1.0, float("inf")), (3e38, 1e-3)])
def test_bad_samples_are_rejected_on_the_host(kappa, tau):
    L = S.lib()
    assert L.nm_mask_forward(_shape(), _sample(kappa, tau), FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_backward(_shape(), _sample(kappa, tau), FAKE, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_backward_wreg(_shape(), _sample(kappa, tau), 0.5, FAKE, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_debug_soft_mask(_shape(), _sample(kappa, tau), FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_forward_monitor(_shape(), _sample(kappa, tau), FAKE, FAKE, FAKE, None, None,
                                     FAKE, FAKE, 1 << 20, None) == NM_EINVAL


def test_null_and_misaligned_pointers_are_rejected_on_the_host():
    L = S.lib()
    sh, sm = _shape(), _sample()
    assert L.nm_mask_forward(None, sm, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_forward(sh, None, FAKE, FAKE, FAKE, None) == NM_EINVAL
    for i in range(3):
        args = [FAKE] * 3
        args[i] = None
        assert L.nm_mask_forward(sh, sm, *args, None) == NM_EINVAL
        args[i] = ODD
        assert L.nm_mask_forward(sh, sm, *args, None) == NM_EALIGN
    for i in range(4):
        args = [FAKE] * 4
        args[i] = None
        assert L.nm_mask_backward(sh, sm, *args, None) == NM_EINVAL
        args[i] = ODD
        assert L.nm_mask_backward(sh, sm, *args, None) == NM_EALIGN
    for i in range(4):
        args = [FAKE] * 4
        args[i] = None
        assert L.nm_mask_harden_pack(sh, *args, None, None) == NM_EINVAL
        args[i] = ODD
        assert L.nm_mask_harden_pack(sh, *args, None, None) == NM_EALIGN
    assert L.nm_mask_harden_pack(sh, FAKE, FAKE, FAKE, FAKE, ODD, None) == NM_EALIGN
    for i in range(3):
        args = [FAKE] * 3
        args[i] = None
        assert L.nm_unpack(sh, *args, None) == NM_EINVAL
        args[i] = ODD
        assert L.nm_unpack(sh, *args, None) == NM_EALIGN
    for i in range(2):
        args = [FAKE] * 2
        args[i] = None
        assert L.nm_prior_init(sh, 3.0, *args, FAKE, None) == NM_EINVAL
        args[i] = ODD
        assert L.nm_prior_init(sh, 3.0, *args, FAKE, None) == NM_EALIGN
    big = 1 << 20
    for i in range(5):   # w, logits, w_masked, stats, workspace
        args = [FAKE] * 5
        args[i] = None
        mon = lambda a: L.nm_mask_forward_monitor(sh, sm, a[0], a[1], a[2], None, None, a[3], a[4], big, None)
        assert mon(args) == NM_EINVAL
        args[i] = ODD
        assert mon(args) == NM_EALIGN
    # prev_sample and sample are optional and need no alignment
    assert L.nm_mask_forward_monitor(sh, sm, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 0, None) == NM_EINVAL
    need = L.nm_monitor_workspace_bytes(sh)
    assert need == 16  # 16 groups of 2:4: one block, no tree above it (the minimum size)
    assert L.nm_mask_forward_monitor(sh, sm, FAKE, FAKE, FAKE, ODD, ODD, FAKE, FAKE, need - 1, None) == NM_EINVAL
    for alpha in (float("nan"), float("inf"), -float("inf")):
        assert L.nm_prior_init(sh, alpha, FAKE, FAKE, None, None) == NM_EINVAL
    assert L.nm_debug_copy(FAKE, FAKE, -16, None) == NM_EINVAL
    assert L.nm_debug_copy(FAKE, FAKE, 24, None) == NM_EINVAL      # not a multiple of 16
    assert L.nm_debug_copy(None, FAKE, 32, None) == NM_EINVAL
    assert L.nm_debug_copy(FAKE, ODD, 32, None) == NM_EALIGN
    assert L.nm_debug_copy(None, None, 0, None) == NM_OK
    assert L.nm_debug_gumbel_log2(FAKE, FAKE, -1, None) == NM_EINVAL
    assert L.nm_debug_gumbel_log2(None, FAKE, 5, None) == NM_EINVAL
    assert L.nm_debug_gumbel_log2(ODD, FAKE, 5, None) == NM_EALIGN


@pytest.mark.parametrize("rows,cols", [(0, 16), (4, 0), (0, 0)])
def test_empty_matrices_are_valid_and_launch_nothing(rows, cols):
    """No pointer is touched (they may be null) and no HIP call is made."""
    L = S.lib()
    sh, sm = _shape(rows=rows, cols=cols), _sample()
    assert L.nm_mask_forward(sh, sm, None, None, None, None) == NM_OK
    assert L.nm_mask_backward(sh, sm, None, None, None, None, None) == NM_OK
    assert L.nm_mask_harden_pack(sh, None, None, None, None, None, None) == NM_OK
    assert L.nm_unpack(sh, None, None, None, None) == NM_OK
    assert L.nm_debug_noise(sh, sm, None, None) == NM_OK
    assert L.nm_debug_soft_mask(sh, sm, None, None, None) == NM_OK
    assert L.nm_debug_gumbel_log2(None, None, 0, None) == NM_OK
    assert L.nm_prior_init(sh, 3.0, None, None, None, None) == NM_OK
    assert L.nm_mask_forward_monitor(sh, sm, None, None, None, None, None, None, None, 0, None) == NM_OK
    assert L.nm_packed_value_elems(sh) == 0


@pytest.mark.parametrize("n,m", SUPPORTED)
def test_candidate_table_and_sizes_agree_with_the_oracle(n, m):
    assert S.num_candidates(n, m) == oracle.num_candidates(n, m)
    assert S.candidate_table(n, m) == list(oracle.candidate_bits(n, m))
    for cols in (m, 8 * m, 13 * m, 4096):
        assert S.index_words_per_row(cols, n, m) == oracle.index_words_per_row(cols, n, m)
        sh = S._Shape(5, cols, n, m, 1)
        assert S.lib().nm_packed_value_elems(ctypes.byref(sh)) == 5 * cols // m * n
        assert S.lib().nm_packed_index_words(ctypes.byref(sh)) == 5 * oracle.index_words_per_row(cols, n, m)


@pytest.mark.parametrize("n,m", SUPPORTED)
def test_monitor_workspace_layout(n, m):
    """Two 8-byte words per node of a 64-ary tree over the launch's blocks of 256 threads, at
    least 16 bytes."""
    K = oracle.num_candidates(n, m)
    P = 1 if (K % 4 == 0 or K == 70) else (2 if K % 2 == 0 else 4)
    for rows, cols in [(1, m), (37, 23 * m), (4096, 4096), (4100, 16384), (70000, 12288)]:
        groups = rows * cols // m
        below, words = -(-(-(-groups // P)) // 256), 0
        while below > 1:
            below = -(-below // 64)
            words += 2 * below
        assert S.monitor_workspace_bytes(rows, cols, n, m) == 8 * max(words, 2)


def test_sparse_matmul_is_validated_on_the_host():
    L = S.lib()
    sh = _shape(rows=256, cols=64, n=2, m=4, wtype=1)
    ok = lambda shp, tokens=256, y=FAKE, ytype=1, v=FAKE: L.nm_sparse_matmul(shp, v, FAKE, FAKE, tokens, y, ytype, None)
    assert ok(_shape(rows=256, cols=64, n=2, m=4, wtype=0)) == NM_EUNSUPPORTED   # fp32 weights
    assert ok(_shape(rows=256, cols=64, n=1, m=4, wtype=1)) == NM_EUNSUPPORTED   # 1:4
    assert ok(_shape(rows=130, cols=64, n=2, m=4, wtype=1)) == NM_EUNSUPPORTED   # out % 4
    assert ok(_shape(rows=256, cols=96, n=2, m=4, wtype=1)) == NM_EUNSUPPORTED   # in % 64
    assert ok(sh, tokens=1 << 40) == NM_EINVAL                                    # grid beyond 2^31 blocks
    assert ok(sh, tokens=-1) == NM_EINVAL
    assert ok(sh, ytype=5) == NM_EINVAL
    assert ok(sh, y=None) == NM_EINVAL
    assert ok(sh, v=ODD) == NM_EALIGN
    assert ok(sh, tokens=0, y=None) == NM_OK
    assert ok(_shape(rows=0, cols=64, n=2, m=4, wtype=1), y=None) == NM_OK


# Plans of the product on 256 compute units (the count taken when no GPU can be asked, and
# MI355X's): each is the candidate measured fastest for that shape on MI355X (graph replays of
# every tile x parts candidate, the weights read from HBM at every call).
PLANS = [
    ((4096, 4096, 1), True, (0, 1)), ((4096, 11008, 4), True, (16, 1)), ((4096, 4096, 16), False, (16, 1)),
    ((11008, 4096, 16), True, (64, 4)), ((4096, 11008, 16), True, (64, 8)), ((4096, 4096, 64), True, (64, 4)),
    ((11008, 4096, 128), True, (128, 2)), ((4096, 11008, 128), True, (128, 8)), ((4096, 4096, 512), True, (128, 2)),
    ((4096, 4096, 768), True, (128, 1)), ((11008, 4096, 1024), True, (256, 1)), ((4096, 11008, 1024), True, (256, 4)),
    ((4096, 11008, 2048), True, (256, 2)), ((4096, 4096, 4096), True, (256, 1)), ((1024, 4096, 64), True, (64, 8)),
    ((4096, 4096, 64), False, (16, 1)), ((4096, 11008, 2048), False, (128, 1)), ((4096, 4096, 256), True, (128, 4)),
    ((4096, 4096, 16), True, (16, 1)),
]


@pytest.mark.parametrize("shape,split,plan", PLANS)
def test_sparse_matmul_plan_and_workspace(shape, split, plan):
    """Without a GPU the plan takes 256 compute units; the workspace is one fp32 [tokens, out]
    slice per part of a split k range, none without a split."""
    out, inn, tokens = shape
    assert S.sparse_matmul_plan(out, inn, tokens, split=split) == plan
    if split:
        parts = plan[1]
        assert S.sparse_matmul_workspace_bytes(out, inn, tokens) == (4 * parts * tokens * out if parts > 1 else 0)


def test_sparse_matmul_plan_bounds():
    """Parts never exceed k's 64-wide stages, no split without a workspace, and a huge product
    still gets a plan whose grid fits (its 256 tiles: what the entry points admit)."""
    for out, inn, tokens in [(4, 64, 100), (4, 128, 100), (260, 192, 300), (8, 24640, 1), (4, 512, 60_000_000_000)]:
        tile, parts = S.sparse_matmul_plan(out, inn, tokens)
        assert tile in (0, 16, 64, 128, 256) and parts in (1, 2, 4, 8) and parts <= inn // 64
        assert S.sparse_matmul_plan(out, inn, tokens, split=False)[1] == 1
    assert S.sparse_matmul_plan(4, 512, 60_000_000_000)[1] == 1          # no split of a 2^41+ output
    assert S.sparse_matmul_plan(256, 64, 0) == (-1, 0)
    # the tallest weight the checks admit (2^35 - 16 rows of 64 columns) still gets a plan; the
    # 16-row kernel's grid is then exactly 2^31 - 1 blocks
    tall = (1 << 35) - 16
    tile, _ = S.sparse_matmul_plan(tall, 64, 64)
    assert tile != 16 or (tall + 15) // 16 <= 2**31 - 1


def test_sparse_matmul_ws_is_validated_on_the_host():
    L = S.lib()
    sh = _shape(rows=4096, cols=4096, n=2, m=4, wtype=1)
    need = L.nm_sparse_matmul_workspace_bytes(sh, 64)
    assert need == 4 * 4 * 64 * 4096                      # 64 tokens: 64 tiles in 4 parts
    call = lambda ws, nbytes, tokens=64, shp=sh: L.nm_sparse_matmul_ws(shp, FAKE, FAKE, FAKE, tokens, FAKE, 1,
                                                                        ws, nbytes, None)
    assert call(None, 0) == NM_EINVAL                     # a split needs the workspace
    assert call(FAKE, need - 16) == NM_EINVAL             # short
    assert call(ODD, need) == NM_EALIGN
    assert call(None, 0, tokens=-1) == NM_EINVAL
    assert call(None, 0, tokens=0) == NM_OK               # empty: nothing to do, no workspace
    assert call(None, 0, shp=_shape(rows=130, cols=64, n=2, m=4, wtype=1)) == NM_EUNSUPPORTED
    assert L.nm_sparse_matmul_workspace_bytes(_shape(rows=130, cols=64, n=2, m=4, wtype=1), 256) == -1
    assert L.nm_sparse_matmul_workspace_bytes(_shape(rows=256, cols=64, n=2, m=4, wtype=0), 256) == -1
    assert L.nm_sparse_matmul_workspace_bytes(sh, -1) == -1
    assert L.nm_sparse_matmul_workspace_bytes(sh, 0) == 0
    assert L.nm_sparse_matmul_workspace_bytes(_shape(rows=0, cols=64, n=2, m=4, wtype=1), 256) == 0


def test_unsupported_helpers():
    assert S.num_candidates(2, 6) == -1 and S.num_candidates(4, 4) == -1
    assert S.lib().nm_candidate_table(2, 6, None) == NM_EUNSUPPORTED
    assert S.lib().nm_candidate_table(2, 4, None) == NM_EINVAL
    assert S.lib().nm_status_str(NM_EALIGN) == b"pointer not 16-byte aligned"


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, 16)
    L = torch.zeros(4, 4, 6)
    with pytest.raises(ValueError):
        S.nm_mask_forward(w, L, 2, 4, 1.0, 1.0, 0, 0)


@pytest.mark.parametrize("lam", [float("nan"), float("inf"), -float("inf"), 3e38])
def test_regulariser_strength_must_be_finite(lam):
    """lambda and 2*lambda must be finite fp32 numbers (3e38 doubles past the fp32 range)."""
    L = S.lib()
    assert L.nm_mask_backward_wreg(_shape(), _sample(), lam, FAKE, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_backward_wreg(_shape(), _sample(), lam, FAKE, FAKE, None, FAKE, None) == NM_EINVAL


def test_regulariser_backward_pointer_rules():
    """grad_w_masked may be NULL (the regulariser alone); every other pointer is required, and
    every non-NULL pointer must be 16-byte aligned.  An empty matrix launches nothing."""
    L = S.lib()
    sh, smp = _shape(), _sample()
    for args in [(None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, FAKE, None)]:
        assert L.nm_mask_backward_wreg(sh, smp, 0.5, *args, None) == NM_EINVAL
    for args in [(ODD, FAKE, FAKE, FAKE), (FAKE, ODD, FAKE, FAKE), (FAKE, FAKE, ODD, FAKE),
                 (FAKE, FAKE, FAKE, ODD), (FAKE, FAKE, None, ODD)]:
        assert L.nm_mask_backward_wreg(sh, smp, 0.5, *args, None) == NM_EALIGN
    assert L.nm_mask_backward_wreg(_shape(rows=0), smp, 0.5, None, None, None, None, None) == NM_OK


def test_forward_pack_pointer_rules():
    """Every pointer but hard_idx is required; all must be 16-byte aligned; a bad sample is
    refused; an empty matrix launches nothing."""
    L = S.lib()
    sh, smp = _shape(), _sample()
    args = [FAKE] * 5
    for i in range(5):
        a = list(args)
        a[i] = None
        assert L.nm_mask_forward_pack(sh, smp, *a, None, None) == NM_EINVAL
        a[i] = ODD
        assert L.nm_mask_forward_pack(sh, smp, *a, None, None) == NM_EALIGN
    assert L.nm_mask_forward_pack(sh, smp, *args, ODD, None) == NM_EALIGN
    assert L.nm_mask_forward_pack(sh, _sample(1.0, 0.0), *args, None, None) == NM_EINVAL
    assert L.nm_mask_forward_pack(_shape(rows=0), smp, None, None, None, None, None, None, None) == NM_OK


def test_device_offset_pointer_rules():
    """The step offset pointer is required and 8-byte aligned; the other pointers follow
    nm_mask_forward / nm_mask_backward; a bad sample is still refused."""
    L = S.lib()
    sh, smp = _shape(), _sample()
    ODD8 = ctypes.c_void_p((1 << 20) + 4)
    assert L.nm_mask_forward_offset_dev(sh, smp, None, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_forward_offset_dev(sh, smp, ODD8, FAKE, FAKE, FAKE, None) == NM_EALIGN
    assert L.nm_mask_forward_offset_dev(sh, smp, ctypes.c_void_p((1 << 20) + 8), FAKE, FAKE, ODD, None) == NM_EALIGN
    assert L.nm_mask_backward_offset_dev(sh, smp, None, FAKE, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_backward_offset_dev(sh, smp, ODD8, FAKE, FAKE, FAKE, FAKE, None) == NM_EALIGN
    assert L.nm_mask_backward_offset_dev(sh, smp, FAKE, FAKE, FAKE, None, FAKE, None) == NM_EINVAL
    assert L.nm_mask_forward_offset_dev(sh, _sample(1.0, 0.0), FAKE, FAKE, FAKE, FAKE, None) == NM_EINVAL
    assert L.nm_mask_backward_offset_dev(_shape(rows=0), smp, None, None, None, None, None, None) == NM_OK


def test_static_monitor_refuses_shapes_past_its_scratch_size():
    """nm_mask_forward_monitor_static checks its fixed array's size on the host, before any HIP
    call: the fake aligned pointers below are never used."""
    L = S.lib()
    rows, cols = 70000, 12288  # 2:4, two groups per thread: 420,000 blocks, a tree of 106 KB
    sh = S._shape(rows, cols, 2, 4, S.NM_BF16)
    assert L.nm_monitor_workspace_bytes(ctypes.byref(sh)) > S.MONITOR_SCRATCH_BYTES
    st = L.nm_mask_forward_monitor_static(ctypes.byref(sh), ctypes.byref(S._sample(100.0, 4.0, 1, 1)), FAKE, FAKE,
                                          FAKE, None, None, FAKE, None)
    assert st == S.NM_ESCRATCH
    assert L.nm_status_str(st).decode().startswith("shape needs more scratch")
    # the largest layer matrices of the model families fit
    for rows, cols, n, m in [(24576, 6144, 2, 4), (24576, 6144, 1, 4), (11008, 4096, 4, 8)]:
        need = L.nm_monitor_workspace_bytes(ctypes.byref(S._shape(rows, cols, n, m, S.NM_BF16)))
        assert need <= S.MONITOR_SCRATCH_BYTES
    small = S._shape(64, 256, 2, 4, S.NM_BF16)
    assert L.nm_mask_forward_monitor_static(ctypes.byref(small), ctypes.byref(S._sample(100.0, 4.0, 1, 1)), FAKE,
                                            FAKE, FAKE, None, None, ODD, None) == NM_EALIGN
