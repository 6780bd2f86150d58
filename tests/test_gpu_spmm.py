"""GPU parity of the product with the packed 2:4 weights (nm_sparse_matmul, gfx950 sparse
matrix cores) against the oracle's binary64 product, within the fp32 accumulation bound; the
weights come from the path's own harden+pack, so the packed form feeds the product unchanged.
Every call goes through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import nm_synth
import oracle
import semi_structured_sparsity_amd as S
from oracle_inputs import oracle_prior
from parity import spmm_check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _packed_layer(out, inn, seed, w_std=0.02):
    w, L, _ = nm_synth.matrix_inputs(out, inn, 2, 4, torch.bfloat16, w_std, seed, logits="prior", device=DEV,
                                     prior=oracle_prior)
    values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
    return w, values, indices


def _check(values, indices, x, y, rows=None, row_begin=0, bf16_out=False):
    """Compare y (GPU, [tokens, out]) with the oracle over W rows row_begin .. + window."""
    vw = values[row_begin:row_begin + rows] if rows else values
    iw = indices[row_begin:row_begin + rows] if rows else indices
    v, i, xc = vw.cpu(), iw.cpu().numpy().view(np.uint32), x.cpu()
    total = values.shape[0]
    ref = oracle.sparse_matmul(v, i, xc, 2, 4, rows=total, row_begin=row_begin)
    ab = oracle.sparse_matmul(v.abs(), i, xc.abs(), 2, 4, rows=total, row_begin=row_begin)
    got = y[:, row_begin:row_begin + ref.shape[1]].double().cpu().numpy()
    n_terms = x.shape[1] // 2
    ratio, bad = spmm_check(got, ref, ab, n_terms, bf16_out)
    return ratio, bad


@pytest.mark.parametrize("out,inn,tokens", [(256, 64, 256), (512, 192, 256), (256, 1024, 512), (768, 640, 768)])
@pytest.mark.parametrize("ytype", [torch.float32, torch.bfloat16])
def test_sparse_matmul_matches_oracle(out, inn, tokens, ytype):
    _say("spmm", out, inn, tokens, ytype)
    _, values, indices = _packed_layer(out, inn, 40 + out + inn, w_std=1.0)
    x = nm_synth.normal((tokens, inn), 1.0, 41, torch.bfloat16, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=ytype)
    ratio, bad = _check(values, indices, x, y, bf16_out=ytype == torch.bfloat16)
    _say("  err/bound", ratio)
    assert bad == 0


@pytest.mark.parametrize("name_index,tokens", [(0, 512), (4, 256), (6, 256), (0, 4096), (6, 2048)])
def test_sparse_matmul_llama7b_shapes_sampled_rows(name_index, tokens):
    """Full LLaMA-7B-shaped weights (q 4096x4096, gate 11008x4096, down 4096x11008); the oracle
    checks three windows of 128 W rows against every token.  The plans: 128 tiles in 2 k parts
    for q at 512 tokens, unsplit for gate at 256, in 4 parts for down at 256 (43 stages each);
    256 tiles in 2 parts for down at 2048 (86 stages each), unsplit for q at 4096."""
    plans = {(0, 512): (128, 2), (4, 256): (128, 1), (6, 256): (128, 4), (0, 4096): (256, 1), (6, 2048): (256, 2)}
    name, out, inn = nm_synth.LLAMA2_7B_LAYER[name_index]
    _say("spmm", name, out, inn, tokens)
    assert S.sparse_matmul_plan(out, inn, tokens) == plans[(name_index, tokens)]
    _, values, indices = _packed_layer(out, inn, nm_synth.input_seed(2, 0, name_index))
    x = nm_synth.normal((tokens, inn), 1.0, 42, torch.bfloat16, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32)
    for rb in (0, out // 2 + 64, out - 128):
        ratio, bad = _check(values, indices, x, y, rows=128, row_begin=rb)
        _say("  rows", rb, "err/bound", ratio)
        assert bad == 0


def test_sparse_matmul_equals_dense_product_of_the_unpacked_weights():
    """The path end to end: harden+pack on the GPU, then the sparse product, against torch's
    dense fp32 product with the unpacked weights (same fp32 bound)."""
    out, inn, tokens = 512, 1024, 512
    _, values, indices = _packed_layer(out, inn, 43, w_std=1.0)
    dense = S.nm_unpack(values, indices, inn, 2, 4)
    x = nm_synth.normal((tokens, inn), 1.0, 44, torch.bfloat16, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32).double()
    dt = dense.double().t().contiguous()
    ref = x.double() @ dt
    ab = x.double().abs() @ dt.abs()
    assert bool(((y - ref).abs() <= (inn // 2) * 2.0**-24 * ab + 1e-30).all())
    # deterministic: the same inputs give the same bits
    assert torch.equal(S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32), y.float())


@pytest.mark.parametrize("out,inn,tokens", [(4, 64, 1), (260, 64, 100), (516, 192, 300), (1028, 128, 513),
                                             (252, 256, 255)])
@pytest.mark.parametrize("ytype", [torch.float32, torch.bfloat16])
def test_sparse_matmul_partial_tiles(out, inn, tokens, ytype):
    """out and tokens not multiples of the tile (64 x 64 at these sizes): the last tiles are
    partial, every output inside matches the oracle and nothing past y's end is written."""
    _say("spmm partial", out, inn, tokens, ytype)
    _, values, indices = _packed_layer(out, inn, 50 + out + tokens, w_std=1.0)
    x = nm_synth.normal((tokens, inn), 1.0, 51, torch.bfloat16, device=DEV)
    buf = torch.full((tokens * out + 4096,), float("nan"), dtype=ytype, device=DEV)
    y = buf[:tokens * out].view(tokens, out)
    S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, out=y)
    ratio, bad = _check(values, indices, x, y, bf16_out=ytype == torch.bfloat16)
    _say("  err/bound", ratio)
    assert bad == 0
    assert bool(buf[tokens * out:].isnan().all())


@pytest.mark.parametrize("out,inn,tokens,tile", [(6148, 128, 2600, 256), (4100, 192, 2049, 256),
                                                  (4000, 320, 1000, 128), (2052, 128, 1100, 128),
                                                  (1092, 256, 700, 64), (68, 64, 65, 64)])
def test_sparse_matmul_each_tile_size_with_ragged_edges(out, inn, tokens, tile):
    """Every tile size of the product (256, 128 and 64 rows and tokens per block) on shapes
    whose last tiles are partial along both sides: windows of W rows (the ragged last one
    included) against every token, and nothing written past y's end.  Fewer k stages than the
    three in flight are covered by inn = 64 and 128.  nm_sparse_matmul itself, which never
    splits k."""
    assert S.sparse_matmul_plan(out, inn, tokens, split=False) == (tile, 1)
    _say("spmm tile", tile, out, inn, tokens)
    _, values, indices = _packed_layer(out, inn, 70 + out + tokens, w_std=1.0)
    x = nm_synth.normal((tokens, inn), 1.0, 71, torch.bfloat16, device=DEV)
    buf = torch.full((tokens * out + 4096,), float("nan"), dtype=torch.float32, device=DEV)
    y = buf[:tokens * out].view(tokens, out)
    S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32, out=y, split=False)
    win = min(132, out)
    for rb in sorted({0, (out // 2) // 4 * 4, out - win}):
        ratio, bad = _check(values, indices, x, y, rows=min(win, out - rb), row_begin=rb)
        _say("  rows", rb, "err/bound", ratio)
        assert bad == 0
    assert bool(buf[tokens * out:].isnan().all())
    assert torch.equal(S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32, split=False), y)


@pytest.mark.parametrize("out,inn,tokens", [(36, 64, 1), (36, 64, 2), (6000, 128, 1), (5000, 4160, 2),
                                             (520, 11008, 2), (8, 24640, 1), (40, 12352, 2), (36, 64, 3),
                                             (1000, 6144, 3), (520, 4096, 4), (40, 6208, 4), (100, 128, 7),
                                             (256, 4160, 32), (68, 192, 33), (132, 256, 64), (64, 320, 65),
                                             (96, 1024, 128), (4, 64, 128)])
@pytest.mark.parametrize("ytype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("split", [False, True])
def test_sparse_matmul_few_tokens(out, inn, tokens, ytype, split):
    """One to four tokens whose X fits in 48 KB run on the row-streaming kernel (several rows per
    wave, rows longer than one pass of the wave, X of 2 x 11008 bf16, three tokens on the
    four-token kernel); 24640 columns at one token, 12352 at two and 6208 at four are just above
    that and run, like the long rows at 32 tokens, on blocks of 16 W rows whose waves split k
    without a workspace, and on 64 x 64 tiles in 8 k parts with one; the small shapes at 7 to 64
    tokens on the 16-row blocks (fewer k blocks than waves), at 65 and 128 tokens on 64 x 64
    tiles.  Every output against the oracle, nothing written past y."""
    _say("spmm few tokens", out, inn, tokens, ytype, split, S.sparse_matmul_plan(out, inn, tokens, split=split))
    _, values, indices = _packed_layer(out, inn, 60 + out + tokens, w_std=1.0)
    x = nm_synth.normal((tokens, inn), 1.0, 61, torch.bfloat16, device=DEV)
    buf = torch.full((tokens * out + 4096,), float("nan"), dtype=ytype, device=DEV)
    y = buf[:tokens * out].view(tokens, out)
    S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, out=y, split=split)
    ratio, bad = _check(values, indices, x, y, bf16_out=ytype == torch.bfloat16)
    _say("  err/bound", ratio)
    assert bad == 0
    assert bool(buf[tokens * out:].isnan().all())
    # deterministic: partial sums (of waves, or of k parts) are added in a fixed order
    assert torch.equal(S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, split=split), y)


@pytest.mark.parametrize("name_index,tokens", [(4, 1), (6, 2), (5, 4), (6, 16), (0, 128)])
def test_sparse_matmul_llama7b_decode_batches(name_index, tokens):
    """Decode-sized batches on full LLaMA-7B-shaped weights, three windows of 128 W rows."""
    name, out, inn = nm_synth.LLAMA2_7B_LAYER[name_index]
    _say("spmm decode", name, out, inn, tokens)
    _, values, indices = _packed_layer(out, inn, nm_synth.input_seed(2, 0, name_index))
    x = nm_synth.normal((tokens, inn), 1.0, 62, torch.bfloat16, device=DEV)
    y = S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32)
    for rb in (0, out // 2 + 64, out - 128):
        ratio, bad = _check(values, indices, x, y, rows=128, row_begin=rb)
        _say("  rows", rb, "err/bound", ratio)
        assert bad == 0


# Exact arithmetic: weights and activations are integers in [-8, 8], so every product (|.| <= 64)
# and every fp32 partial sum (at most 5,504 kept terms here, |.| < 2^19) is exact in any order.
# The product must then equal the oracle's binary64 result bit for bit (and its bf16 rounding,
# round-to-nearest-even, for bf16 outputs): one dropped, repeated or misplaced kept value
# anywhere changes an output.  Each shape runs without a workspace (nm_sparse_matmul) and with
# one (nm_sparse_matmul_ws).  The shapes take every kernel: the row-streaming kernel at 1-4
# tokens (several rows per wave, rows longer than one pass, a partial last pass); the 16-row
# kernel for one, two and four token groups (5-16, 17-32 and 33-64 tokens) and just above the
# streaming kernel's X limit; the 64, 128 and 256 tiles with ragged edges, unsplit and split.
EXACT_SHAPES = [
    (36, 64, 1), (6000, 128, 1), (520, 11008, 2), (36, 64, 3), (1000, 6144, 3), (520, 4096, 4),  # streaming
    (8, 24640, 1), (40, 12352, 2), (40, 6208, 4), (40, 576, 5), (256, 4160, 16), (40, 1088, 17),  # 16-row
    (256, 4160, 32), (40, 1088, 33), (516, 1088, 17), (2052, 1088, 33),
    (100, 128, 7), (68, 192, 17), (68, 192, 33), (132, 256, 64),  # 16-row, fewer k blocks than waves
    (260, 64, 100), (1092, 256, 700),  # 64 x 64 tiles
    (2052, 128, 1100), (4000, 320, 1000),  # 128 x 128
    (4100, 192, 2049), (6148, 128, 2600),  # 256 x 256
]


@pytest.mark.parametrize("out,inn,tokens", EXACT_SHAPES)
@pytest.mark.parametrize("ytype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("split", [False, True])
def test_sparse_matmul_exact_on_small_integers(out, inn, tokens, ytype, split):
    _say("spmm exact", out, inn, tokens, ytype, split, S.sparse_matmul_plan(out, inn, tokens, split=split))
    w = nm_synth.small_integers((out, inn), 8, 80 + out + tokens, device=DEV)
    L = nm_synth.gaussian_logits(out, inn, 2, 4, 81 + out, device=DEV)
    values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
    x = nm_synth.small_integers((tokens, inn), 8, 82 + inn + tokens, device=DEV)
    buf = torch.full((tokens * out + 4096,), float("nan"), dtype=ytype, device=DEV)
    y = buf[:tokens * out].view(tokens, out)
    S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, out=y, split=split)
    ref = oracle.sparse_matmul(values.cpu(), indices.cpu().numpy().view(np.uint32), x.cpu(), 2, 4)
    assert np.all(np.abs(ref) < 2**24) and np.array_equal(ref, np.round(ref))  # exact integers
    want = torch.from_numpy(ref).to(torch.float32).to(ytype)
    got = y.cpu()
    bits = (lambda t: t.view(torch.int16)) if ytype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    wrong = int((bits(got) != bits(want)).sum())
    assert wrong == 0, f"{wrong} outputs differ from the exact product"
    assert bool(buf[tokens * out:].isnan().all())


# Split k (nm_sparse_matmul_ws): shapes whose plan is each tile split into each number of parts,
# with ragged last tiles along both sides and parts of unequal length (k stages 7 x 1 + 2,
# 3 x 4 + 5, 8 + 9, 3 x 8 + 9, 7 x 4 + 5, 3 x 16 + 17, 32 + 33), shapes where the 16-row kernel
# stays the cheapest with a workspace (one with a single k stage), and LLaMA-7B-shaped matrices
# at batch sizes where the split is taken (and one where it is not).
SPLIT_SHAPES = [
    (68, 576, 65, 64, 8), (1092, 1088, 65, 64, 4), (2052, 1088, 65, 64, 2), (8196, 1088, 65, 128, 2),
    (4100, 2112, 65, 128, 4), (2052, 2112, 65, 128, 8), (8196, 4160, 130, 256, 4), (2052, 4160, 2049, 256, 2),
    (68, 64, 5, 16, 1), (2052, 1088, 33, 16, 1),
    (4096, 4096, 64, 64, 4), (4096, 4096, 128, 64, 2), (4096, 4096, 256, 128, 4), (4096, 11008, 128, 128, 8),
    (11008, 4096, 1024, 256, 1),
]


def _oracle_rows(values, indices, x, row_begin, rows):
    return oracle.sparse_matmul(values[row_begin:row_begin + rows].cpu(),
                                indices[row_begin:row_begin + rows].cpu().numpy().view(np.uint32), x.cpu(), 2, 4,
                                rows=values.shape[0], row_begin=row_begin)


@pytest.mark.parametrize("out,inn,tokens,tile,parts", SPLIT_SHAPES)
@pytest.mark.parametrize("ytype", [torch.float32, torch.bfloat16])
def test_sparse_matmul_split_k_exact_on_small_integers(out, inn, tokens, tile, parts, ytype):
    """Integer weights and activations in [-8, 8] keep every partial sum exact (|.| < 2^19 here),
    so the parts' sums added in any order give the exact product: every output of the split
    product equals the unsplit one bit for bit, and W-row windows (all rows when the oracle is
    quick) equal the oracle's binary64 product (bf16: its round-to-nearest-even).  The workspace
    is filled with NaN first (its contents on entry must not matter) and nothing past y is
    written."""
    assert S.sparse_matmul_plan(out, inn, tokens) == (tile, parts)
    _say("spmm split", out, inn, tokens, tile, parts, ytype)
    need = S.sparse_matmul_workspace_bytes(out, inn, tokens)
    assert need == (4 * parts * tokens * out if parts > 1 else 0)
    w = nm_synth.small_integers((out, inn), 8, 90 + out + tokens, device=DEV)
    L = nm_synth.gaussian_logits(out, inn, 2, 4, 91 + out, device=DEV)
    values, indices = S.nm_mask_harden_pack(w, L, 2, 4)
    x = nm_synth.small_integers((tokens, inn), 8, 92 + inn + tokens, device=DEV)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV).view(torch.uint8)
    buf = torch.full((tokens * out + 4096,), float("nan"), dtype=ytype, device=DEV)
    y = buf[:tokens * out].view(tokens, out)
    S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, out=y, workspace=ws)
    plain = S.nm_sparse_matmul(values, indices, x, out_dtype=ytype, split=False)
    bits = (lambda t: t.view(torch.int16)) if ytype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(y), bits(plain))
    assert bool(buf[tokens * out:].isnan().all())
    windows = [(0, out)] if out * inn * tokens <= 2**30 else [(0, 128), ((out // 2) // 4 * 4, 128), (out - 132, 132)]
    for rb, nr in windows:
        ref = _oracle_rows(values, indices, x, rb, nr)
        assert np.all(np.abs(ref) < 2**24) and np.array_equal(ref, np.round(ref))  # exact integers
        want = torch.from_numpy(ref).to(torch.float32).to(ytype)
        wrong = int((bits(y[:, rb:rb + nr].cpu()) != bits(want)).sum())
        assert wrong == 0, f"rows {rb}..: {wrong} outputs differ from the exact product"


def test_sparse_matmul_split_k_workspace_reuse_and_size_check():
    """One workspace serves calls in a row, the second on a smaller batch (its leftovers from the
    first call do not leak into the second's outputs); a workspace one float short is refused
    before anything runs, and y is left as it was."""
    out, inn = 4096, 4096
    _, values, indices = _packed_layer(out, inn, nm_synth.input_seed(2, 0, 0))
    big, small = 512, 128
    need = S.sparse_matmul_workspace_bytes(out, inn, big)
    assert need > 0 and S.sparse_matmul_workspace_bytes(out, inn, small) <= need
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for tokens in (big, small):
        _say("spmm split reuse", tokens)
        x = nm_synth.normal((tokens, inn), 1.0, 95 + tokens, torch.bfloat16, device=DEV)
        y = S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32, workspace=ws)
        for rb in (0, out - 128):
            ratio, bad = _check(values, indices, x, y, rows=128, row_begin=rb)
            _say("  rows", rb, "err/bound", ratio)
            assert bad == 0
        # deterministic: the parts are added in a fixed order
        assert torch.equal(S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32, workspace=ws), y)
    x = nm_synth.normal((big, inn), 1.0, 96, torch.bfloat16, device=DEV)
    y = torch.full((big, out), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(S.NMError) as e:
        S.nm_sparse_matmul(values, indices, x, out_dtype=torch.float32, out=y, workspace=ws[:need - 4])
    assert e.value.status == S.NM_EINVAL
    assert bool((y == 7.0).all())


def test_sparse_matmul_rejects_unsupported_shapes():
    _, values, indices = _packed_layer(256, 64, 45)
    x = torch.zeros((128, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(S.NMError) as e:
        S.nm_sparse_matmul(values[:254], indices[:254], x)   # out not a multiple of 4
    assert e.value.status == S.NM_EUNSUPPORTED
    x0 = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    assert S.nm_sparse_matmul(values, indices, x0).shape == (0, 256)
