"""Calls on two streams at once.  The entry points keep no state between calls (the noise is a
function of the arguments, and each call's scratch is its caller's workspace), so the same calls
issued alternately on two non-default streams, with nothing ordering one stream against the
other, give the outputs of the same calls made one after another on the default stream, bit for
bit; monitored forwards and split products with one workspace per stream give the same samples,
stats and products.  Every call goes through the C ABI."""
import sys

import pytest
import torch

import nm_synth
import semi_structured_sparsity_amd as S

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPES = [(2048, 4096), (4096, 1024), (1024, 4096), (512, 11008)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) if t.is_floating_point() else t


def _calls(w, L, G, n, m, i):
    fwd = S.nm_mask_forward(w, L, n, m, 100.0, 4.0, 40 + i, 3)
    bwd = S.nm_mask_backward(w, L, G, n, m, 100.0, 4.0, 40 + i, 3)
    values, indices, hard = S.nm_mask_harden_pack(w, L, n, m, with_hard=True)
    dense = S.nm_unpack(values, indices, w.shape[1], n, m)
    return fwd, bwd, values, indices, hard, dense


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_two_streams_give_the_serial_outputs(n, m):
    _say("streams", n, m)
    mats = [nm_synth.matrix_inputs(r, c, n, m, torch.bfloat16, 0.02, 60 + i, device=DEV)
            for i, (r, c) in enumerate(SHAPES)]
    refs = [_calls(w, L, G, n, m, i) for i, (w, L, G) in enumerate(mats)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        outs = []
        for i, (w, L, G) in enumerate(mats):
            with torch.cuda.stream(streams[i % 2]):
                outs.append(_calls(w, L, G, n, m, i))
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, refs)):
            for k, (a, b) in enumerate(zip(got, ref)):
                assert torch.equal(_bits(a), _bits(b)), f"rep {rep} matrix {i} output {k}"


def test_monitored_forwards_on_two_streams_with_their_own_workspaces():
    n, m = 2, 4
    _say("streams monitor")
    mats = [nm_synth.matrix_inputs(r, c, n, m, torch.bfloat16, 0.02, 70 + i, with_grad=False, device=DEV)
            for i, (r, c) in enumerate(SHAPES)]
    need = max(S.monitor_workspace_bytes(r, c, n, m) for r, c in SHAPES)
    prev = [torch.randint(0, 7, (r, c // m), dtype=torch.uint8, device=DEV) for r, c in SHAPES]
    refs = [S.nm_mask_forward_monitor(w, L, n, m, 100.0, 4.0, 9, i, prev_sample=prev[i])
            for i, (w, L, _) in enumerate(mats)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    spaces = [torch.zeros(need, dtype=torch.uint8, device=DEV) for _ in streams]
    torch.cuda.synchronize()
    for rep in range(3):
        outs = []
        for i, (w, L, _) in enumerate(mats):
            with torch.cuda.stream(streams[i % 2]):
                outs.append(S.nm_mask_forward_monitor(w, L, n, m, 100.0, 4.0, 9, i, prev_sample=prev[i],
                                                      workspace=spaces[i % 2]))
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(got[0]), _bits(ref[0])), f"rep {rep} matrix {i} w_masked"
            assert torch.equal(got[1], ref[1]), f"rep {rep} matrix {i} samples"
            assert torch.equal(got[2], ref[2]), f"rep {rep} matrix {i} stats"
    assert not any(bool(s.any()) for s in spaces)  # every call left its workspace zero


def test_split_products_on_two_streams():
    """Products whose plans split k (LLaMA-7B-shaped weights at 64 to 256 tokens), issued
    alternately on two streams: with one workspace per stream, given by the caller, and with the
    binding's own per-call workspaces, every output equals that of the same call made alone."""
    _say("streams spmm")
    cases = [(4096, 4096, 64), (11008, 4096, 128), (4096, 11008, 256), (4096, 4096, 256)]
    mats = []
    for i, (out, inn, tokens) in enumerate(cases):
        assert S.sparse_matmul_plan(out, inn, tokens)[1] > 1
        w, L, _ = nm_synth.matrix_inputs(out, inn, 2, 4, torch.bfloat16, 0.02, 80 + i, with_grad=False, device=DEV)
        values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
        x = nm_synth.normal((tokens, inn), 1.0, 90 + i, torch.bfloat16, device=DEV)
        mats.append((values, indices, x))
    refs = [S.nm_sparse_matmul(v, ix, x) for v, ix, x in mats]
    torch.cuda.synchronize()
    need = max(S.sparse_matmul_workspace_bytes(out, inn, tokens) for out, inn, tokens in cases)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    spaces = [torch.empty(need, dtype=torch.uint8, device=DEV) for _ in streams]
    torch.cuda.synchronize()
    for own in (True, False):
        for rep in range(3):
            outs = []
            for i, (v, ix, x) in enumerate(mats):
                with torch.cuda.stream(streams[i % 2]):
                    outs.append(S.nm_sparse_matmul(v, ix, x, workspace=spaces[i % 2] if own else None))
            torch.cuda.synchronize()
            for i, (got, ref) in enumerate(zip(outs, refs)):
                assert torch.equal(_bits(got), _bits(ref)), f"own workspace {own} rep {rep} product {i}"
