"""The entry points can be captured into a HIP graph (through torch's graph capture on the
current stream): they allocate nothing, synchronise nothing and record no memset.  Each graph is
replayed several times with eager work and synchronisations between the replays, and every
replay's outputs are compared bit for bit with the eager call's (same arguments, so the same
noise).  Every call goes through the C ABI."""
import sys

import pytest
import torch

import nm_synth
import semi_structured_sparsity_amd as S
from oracle_inputs import oracle_prior

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) if t.is_floating_point() else t


def _replay_and_compare(graph, outs, refs, reps=3):
    for r in range(reps):
        for o in outs:  # poison the outputs: a replay that writes nothing cannot pass
            if o.is_floating_point():
                o.fill_(float("nan"))
            else:
                o.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        scratch = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for o, ref in zip(outs, refs):
            assert torch.equal(_bits(o), _bits(ref)), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("shape,wtype", [((256, 256), torch.float32), ((4096, 4096), torch.bfloat16)])
def test_layer_step_replays_as_a_graph(shape, wtype):
    n, m, kappa, tau, seed, off = 2, 4, 100.0, 4.0, 5, 7
    rows, cols = shape
    _say("graph step", shape, wtype)
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, wtype, 0.02, 3, logits="prior", prior=oracle_prior,
                                     device=DEV)
    out, dl = torch.empty_like(w), torch.empty_like(L)
    values = torch.empty((rows, cols // 2), dtype=wtype, device=DEV)
    indices = torch.empty((rows, cols // 32), dtype=torch.int32, device=DEV)
    dense = torch.empty_like(w)

    def step():
        S.nm_mask_forward(w, L, n, m, kappa, tau, seed, off, out=out)
        S.nm_mask_backward(w, L, G, n, m, kappa, tau, seed, off, out=dl)
        S.nm_mask_harden_pack(w, L, n, m, out=(values, indices, None))
        S.nm_unpack(values, indices, cols, n, m, out=dense)

    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in (out, dl, values, indices, dense)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    _replay_and_compare(g, [out, dl, values, indices, dense], refs)


@pytest.mark.parametrize("tokens", [1, 3, 16, 256])
def test_sparse_product_replays_as_a_graph(tokens):
    """Decode- and prefill-sized products of a packed LLaMA-7B-shaped weight (4096x4096)."""
    _say("graph spmm", tokens)
    w, L, _ = nm_synth.matrix_inputs(4096, 4096, 2, 4, torch.bfloat16, 0.02, 4, device=DEV)
    values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
    x = nm_synth.normal((tokens, 4096), 1.0, 5, torch.bfloat16, device=DEV)
    y = torch.empty((tokens, 4096), dtype=torch.bfloat16, device=DEV)
    S.nm_sparse_matmul(values, indices, x, out=y)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        S.nm_sparse_matmul(values, indices, x, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.nm_sparse_matmul(values, indices, x, out=y)
    _replay_and_compare(g, [y], [ref])


@pytest.mark.parametrize("wtype", [torch.bfloat16, torch.float32])
def test_training_step_graph_with_the_offset_on_the_device(wtype):
    """A forward + backward captured once, with the step offset read from a device tensor, and
    replayed for steps 3, 4, 11 and 2**40 + 5: each replay equals the eager calls at that step
    (fresh noise per replay), bit for bit."""
    n, m, kappa, tau, seed = 2, 4, 100.0, 4.0, 21
    rows, cols = 96, 512
    _say("graph device offset", wtype)
    w, L, G = nm_synth.matrix_inputs(rows, cols, n, m, wtype, 0.5, 22, device=DEV)
    step = torch.zeros(1, dtype=torch.int64, device=DEV)
    out, dl = torch.empty_like(w), torch.empty_like(L)

    def run():
        S.nm_mask_forward(w, L, n, m, kappa, tau, seed, step, out=out)
        S.nm_mask_backward(w, L, G, n, m, kappa, tau, seed, step, out=dl)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    prev = None
    for k in (3, 4, 11, 2**40 + 5):
        step.fill_(k)
        out.fill_(float("nan"))
        dl.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_f = S.nm_mask_forward(w, L, n, m, kappa, tau, seed, k)
        ref_b = S.nm_mask_backward(w, L, G, n, m, kappa, tau, seed, k)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_f)), f"forward replay at step {k}"
        assert torch.equal(_bits(dl), _bits(ref_b)), f"backward replay at step {k}"
        if prev is not None:
            assert not torch.equal(_bits(out), prev), "each step samples fresh noise"
        prev = _bits(out).clone()


@pytest.mark.parametrize("n,m,shape", [(2, 4, (4096, 4096)), (4, 8, (520, 1024)), (1, 4, (4100, 16384))])
def test_monitored_forward_replays_as_a_graph(n, m, shape):
    """The monitored forward in one graph node: the stats are summed inside the launch through
    counters in the workspace, which every launch leaves at zero, so each replay sums afresh.
    (4100 x 16384 at 1:4 is 65,600 blocks: a tree of three levels above them.)"""
    rows, cols = shape
    _say("graph monitor", n, m, shape)
    w, L, _ = nm_synth.matrix_inputs(rows, cols, n, m, torch.bfloat16, 0.5, 9, with_grad=False, device=DEV)
    g_shape = (rows, cols // m)
    prev = torch.randint(0, S.num_candidates(n, m) + 1, g_shape, dtype=torch.uint8, device=DEV)
    ws = torch.zeros(S.monitor_workspace_bytes(rows, cols, n, m), dtype=torch.uint8, device=DEV)
    out = (torch.empty_like(w), torch.empty(g_shape, dtype=torch.uint8, device=DEV),
           torch.zeros(2, dtype=torch.float64, device=DEV))

    def step():
        S.nm_mask_forward_monitor(w, L, n, m, 30.0, 0.5, 5, 8, prev_sample=prev, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in out]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert all(torch.equal(_bits(o), _bits(r)) for o, r in zip(out, refs))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    _replay_and_compare(g, list(out), refs)
