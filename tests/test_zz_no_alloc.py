"""The monitored forward with no workspace (nm_mask_forward_monitor_static, for callers that
cannot allocate) against the workspace entry point (nm_mask_forward_monitor) through the C ABI:
the same kernels, so every output is bit-identical -- masked weights, sampled candidates and
both sums -- on two calls in a row, the second with a smaller input than the first (the shared
array keeps the first call's partial sums and must not leak them into the second)."""
import sys

import pytest
import torch

import nm_synth
import semi_structured_sparsity_amd as S

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(w, L, n, m, kappa, tau, seed, offset, prev):
    ref = S.nm_mask_forward_monitor(w, L, n, m, kappa, tau, seed, offset, prev_sample=prev)
    got = S.nm_mask_forward_monitor_static(w, L, n, m, kappa, tau, seed, offset, prev_sample=prev)
    torch.cuda.synchronize()
    return ref, got


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_static_scratch_equals_workspace_on_two_calls(n, m):
    # first call: a LLaMA-7B-shaped 11008 x 4096 matrix (22,016 blocks of partial sums); second:
    # a small ragged one, so the array still holds the first call's sums beyond what it needs
    shapes = [(11008, 4096), (37, 23 * m)]
    prev = None
    for i, (rows, cols) in enumerate(shapes):
        _say("static monitor", n, m, rows, cols)
        w, L, _ = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.02, 700 + 10 * m + i, with_grad=False,
                                         device=DEV)
        if i == 1:
            prev = torch.randint(0, nm_synth.num_candidates(n, m) + 1, (rows, cols // m), dtype=torch.uint8,
                                 device=DEV)
        (rw, rs, rst), (gw, gs, gst) = _both(w, L, n, m, 100.0, 4.0, 31, 5 + i, prev)
        assert torch.equal(_bits(gw), _bits(rw))
        assert torch.equal(gs, rs)
        assert torch.equal(gst.view(torch.int64), rst.view(torch.int64)), (gst, rst)
        assert float(gst[0]) > 0.0
