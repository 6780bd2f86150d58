"""Pins of the oracle's hard mask and compressed 2:4 / N:M storage.

"Accelerating Sparse Deep Neural Networks" summary page, section 3.1: the compressed format
stores the kept values only, with 2 bits of metadata per kept value naming its position in the
group of four, and saves about 44% (16-bit) / 38% (8-bit) of storage (tests/golden fixture).
The hard mask is the mode of the learned distribution (first maximum of the logits).
"""
import itertools
import os

import numpy as np
import pytest
import torch

import nm_synth
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
NM = [(2, 4), (1, 4), (3, 4), (1, 8), (2, 8), (4, 8), (7, 8)]


def _bits_per_field(m):
    return (m - 1).bit_length()


def _expected_words(positions, n, m):
    """Reference bitstream built with Python integers: field f at bit f*bits."""
    b = _bits_per_field(m)
    value = 0
    for f, p in enumerate(positions):
        value |= int(p) << (f * b)
    nwords = (len(positions) * b + 31) // 32
    return [(value >> (32 * i)) & 0xFFFFFFFF for i in range(nwords)]


def test_harden_is_first_argmax_brute_force():
    rng = np.random.default_rng(0)
    L = rng.standard_normal((16, 32, 6)).astype(np.float32)
    L[0, 0] = 1.0                       # all tied -> candidate 0
    L[0, 1] = [0, 2, 2, 1, 2, 0]        # tie among 1, 2, 4 -> 1
    L[0, 2] = [-np.inf] * 5 + [-1]      # infinities compare normally
    hard = oracle.harden(L, 2, 4)
    for r, q in itertools.product(range(16), range(32)):
        lst = list(L[r, q])
        assert hard[r, q] == lst.index(max(lst))
    np.testing.assert_array_equal(hard, np.argmax(L, axis=-1))  # numpy's first-max argmax


def test_harden_nan_never_displaces_candidate_zero():
    L = np.array([[[np.nan, 1, 2, 3, 4, 5], [1, np.nan, 0, 0, 2, 0]]], np.float32)
    hard = oracle.harden(L, 2, 4)
    assert hard[0, 0] == 0   # every comparison with the NaN at 0 is false
    assert hard[0, 1] == 4   # a NaN elsewhere is skipped


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_pack_values_and_indices_brute_force(n, m, wtype):
    rows, cols = 5, m * 13   # 13 groups per row: the last index word is partly used
    w = nm_synth.normal((rows, cols), 1.0, 1, wtype)
    L = nm_synth.gaussian_logits(rows, cols, n, m, 2)
    values, idx, hard = oracle.pack(w, L, n, m)
    cand = [c for c in itertools.combinations(range(m), n)]
    wn = oracle._np(w)
    assert values.shape == (rows, cols // m * n)
    assert idx.shape == (rows, oracle.index_words_per_row(cols, n, m))
    for r in range(rows):
        positions = []
        for q in range(cols // m):
            k = int(np.argmax(L[r, q].numpy()))
            assert hard[r, q] == k
            for t, p in enumerate(cand[k]):
                assert values[r, q * n + t] == wn[r, q * m + p]  # bit copy
                positions.append(p)
        assert list(idx[r]) == _expected_words(positions, n, m)


def test_pack_2of4_index_word_by_hand():
    """Eight groups choosing candidates 0,1,2,3,4,5,5,0: positions (0,1),(0,2),(0,3),(1,2),
    (1,3),(2,3),(2,3),(0,1); each group is a nibble p0 | p1 << 2, group q at bits 4q..4q+3:
    nibbles 4,8,C,9,D,E,E,4 from the low end, i.e. the word 0x4EED9C84."""
    L = np.full((1, 8, 6), -1.0, np.float32)
    for q, k in enumerate([0, 1, 2, 3, 4, 5, 5, 0]):
        L[0, q, k] = 1.0
    w = np.arange(32, dtype=np.float32).reshape(1, 32)
    values, idx, _ = oracle.pack(w, L, 2, 4)
    assert idx.tolist() == [[0x4EED9C84]]
    assert values[0].tolist() == [0, 1, 4, 6, 8, 11, 13, 14, 17, 19, 22, 23, 26, 27, 28, 29]


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_unpack_of_pack_is_the_selected_dense_matrix(n, m, wtype):
    rows, cols = 7, m * 11
    w = nm_synth.normal((rows, cols), 1.0, 3, wtype)
    w[0, :m] = -0.0                     # signed zeros that are kept must survive
    L = nm_synth.gaussian_logits(rows, cols, n, m, 4)
    values, idx, hard = oracle.pack(w, L, n, m)
    dense = oracle.unpack(values, idx, cols, n, m)
    mat = oracle.candidate_matrix(n, m).astype(bool)
    keep = mat[hard].reshape(rows, cols)
    wn = oracle._np(w)
    want = np.where(keep, wn, np.zeros_like(wn))   # +0.0 bits where dropped
    assert dense.tobytes() == want.tobytes()
    assert keep.reshape(rows, -1, m).sum(-1).min() == n == keep.reshape(rows, -1, m).sum(-1).max()


@pytest.mark.parametrize("n,m", NM)
def test_index_fields_are_ascending_positions_inside_the_group(n, m):
    rows, cols = 3, m * 40
    L = nm_synth.gaussian_logits(rows, cols, n, m, 5)
    w = nm_synth.normal((rows, cols), 1.0, 6)
    _, idx, _ = oracle.pack(w, L, n, m)
    b = _bits_per_field(m)
    for r in range(rows):
        value = sum(int(v) << (32 * i) for i, v in enumerate(idx[r]))
        fields = [(value >> (f * b)) & ((1 << b) - 1) for f in range(cols // m * n)]
        for q in range(cols // m):
            grp = fields[q * n:(q + 1) * n]
            assert all(0 <= p < m for p in grp)
            assert all(a < c for a, c in zip(grp, grp[1:]))
        assert value >> (len(fields) * b) == 0   # padding bits are zero


def test_packed_size_matches_the_pages_storage_saving():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "storage_savings.txt"))
            if l.strip() and not l.startswith("#")]
    cols = 4096
    words = oracle.index_words_per_row(cols, 2, 4)
    for bits, saving in ((int(a), int(b)) for a, b in rows):
        dense = cols * bits / 8
        packed = cols // 2 * bits / 8 + words * 4
        assert round(100 * (1 - packed / dense)) == saving
    # exactly 0.5625 of the dense bf16 bytes
    assert (cols // 2 * 2 + words * 4) / (cols * 2) == 0.5625


def test_prior_initialised_logits_harden_to_the_prior():
    """Prior-initialised inputs: logit 3 on the oracle's prior candidate plus N(0, 0.1) noise;
    the hard mask of such logits is the prior mask itself."""
    w = nm_synth.normal((6, 64), 0.02, 7, torch.bfloat16)
    for n, m in [(2, 4), (1, 4), (4, 8), (2, 8)]:
        _, idx = oracle.prior_init(w, n, m)
        L = nm_synth.prior_logits(torch.from_numpy(idx.astype(np.int64)), oracle.num_candidates(n, m), seed=1)
        np.testing.assert_array_equal(oracle.harden(L, n, m), idx)


# --- magnitude prior (the step before the path) ----------------------------------------------

def _brute_prior(group, n):
    """The n largest magnitudes; equal magnitudes keep the lower position (stable ranking)."""
    return tuple(sorted(sorted(range(len(group)), key=lambda j: (-abs(group[j]), j))[:n]))


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("wtype", [torch.float32, torch.bfloat16])
def test_prior_init_keeps_the_largest_magnitudes(n, m, wtype):
    rows, cols = 6, m * 24
    w = nm_synth.normal((rows, cols), 0.02, 11, wtype)
    w[0, :m] = 0.5                                   # all tied
    w[1, :m] = torch.tensor([0.5, -0.5] * (m // 2))  # tied magnitudes, opposite signs
    w[2, :m] = 0.0
    w[2, 1] = -0.0                                   # -0.0 and +0.0 have equal magnitude
    logits, idx = oracle.prior_init(w, n, m, alpha=2.5)
    cand = list(itertools.combinations(range(m), n))
    a = w.float().numpy()
    for r in range(rows):
        for q in range(cols // m):
            keep = _brute_prior(list(a[r, q * m:(q + 1) * m]), n)
            k = cand.index(keep)
            assert idx[r, q] == k
            want = np.zeros(len(cand), np.float32)
            want[k] = 2.5
            assert logits[r, q].tobytes() == want.tobytes()
    # and its logits are exactly alpha * onehot
    assert set(np.unique(logits)) <= {0.0, 2.5}


def test_prior_init_nan_rule():
    """A NaN magnitude is taken only as the first unchosen position (no comparison favours it)."""
    w = torch.tensor([[float("nan"), 1.0, 2.0, 3.0, 1.0, float("nan"), 2.0, 0.5]])
    _, idx = oracle.prior_init(w, 2, 4)
    cand = list(itertools.combinations(range(4), 2))
    assert cand[idx[0, 0]] == (0, 3)   # NaN first, then the largest of the rest
    assert cand[idx[0, 1]] == (0, 2)   # 1.0 first (NaN never beats it), then 2.0


def test_prior_init_windows_match_the_whole_matrix():
    w = nm_synth.normal((9, 64), 1.0, 12, torch.bfloat16)
    full_l, full_i = oracle.prior_init(w, 2, 4)
    win_l, win_i = oracle.prior_init(w[3:7], 2, 4, rows=9, row_begin=3)
    np.testing.assert_array_equal(win_l, full_l[3:7])
    np.testing.assert_array_equal(win_i, full_i[3:7])
