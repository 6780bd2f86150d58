"""Pins of the oracle's product with the compressed weights ("Accelerating Sparse Deep Neural
Networks" summary page, sections 3.1-3.2: the sparse operand stays compressed, kept values plus
positions, and multiplies a dense operand).

Pins used: numpy's matmul (a library routine) of X with the transpose of the unpacked weights,
brute force over a dense W rebuilt in Python from the values and a big-integer reading of the
index stream, the identity matrix (Y = W^T exactly), linearity, and row windows.
"""
import itertools

import numpy as np
import pytest
import torch

import nm_synth
import oracle

NM = [(2, 4), (1, 4), (3, 4), (2, 8), (4, 8)]


def _packed(rows, cols, n, m, seed, wtype=torch.bfloat16):
    w = nm_synth.normal((rows, cols), 1.0, seed, wtype)
    L = nm_synth.gaussian_logits(rows, cols, n, m, seed + 1)
    values, indices, _ = oracle.pack(w, L, n, m)
    return w, values, indices


def _dense_from_stream(values, indices, cols, n, m):
    """W rebuilt from the packed form with Python integers: field f of a row at bit f*b."""
    b = (m - 1).bit_length()
    vals = oracle._np(values)
    if vals.dtype == np.uint16:
        vals = (vals.astype(np.uint32) << 16).view(np.float32)
    rows = vals.shape[0]
    W = np.zeros((rows, cols))
    for r in range(rows):
        stream = sum(int(wd) << (32 * i) for i, wd in enumerate(indices[r]))
        for q in range(cols // m):
            for u in range(n):
                f = q * n + u
                p = (stream >> (f * b)) & ((1 << b) - 1)
                W[r, q * m + p] = vals[r, q * n + u]
    return W


@pytest.mark.parametrize("n,m", NM)
@pytest.mark.parametrize("xtype", [torch.float32, torch.bfloat16])
def test_sparse_matmul_matches_library_matmul_of_the_unpacked_weights(n, m, xtype):
    rows, cols, tokens = 9, 16 * m, 13
    w, values, indices = _packed(rows, cols, n, m, 3)
    x = nm_synth.normal((tokens, cols), 1.0, 5, xtype)
    y = oracle.sparse_matmul(values, indices, x, n, m)
    dense = oracle.unpack(values, indices, cols, n, m)
    dense = oracle._np(dense)
    if dense.dtype == np.uint16:
        dense = (dense.astype(np.uint32) << 16).view(np.float32)
    want = x.double().numpy() @ dense.astype(np.float64).T
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,m", NM)
def test_sparse_matmul_brute_force(n, m):
    rows, cols, tokens = 4, 4 * m, 3
    w, values, indices = _packed(rows, cols, n, m, 7)
    x = nm_synth.normal((tokens, cols), 1.0, 8, torch.float32)
    W = _dense_from_stream(values, indices, cols, n, m)
    X = x.double().numpy()
    y = oracle.sparse_matmul(values, indices, x, n, m)
    for t in range(tokens):
        for o in range(rows):
            acc = 0.0
            for i in range(cols):
                acc += X[t, i] * W[o, i]
            assert y[t, o] == pytest.approx(acc, rel=1e-13, abs=1e-13)
    # every row keeps exactly n of every m
    assert ((W.reshape(rows, cols // m, m) != 0).sum(-1) <= n).all()


@pytest.mark.parametrize("n,m", [(2, 4), (3, 8)])
def test_identity_activations_give_the_transposed_weights(n, m):
    rows, cols = 6, 8 * m
    _, values, indices = _packed(rows, cols, n, m, 9, torch.float32)
    eye = torch.eye(cols)
    y = oracle.sparse_matmul(values, indices, eye, n, m)
    W = _dense_from_stream(values, indices, cols, n, m)
    np.testing.assert_array_equal(y, W.T)


def test_sparse_matmul_is_linear_and_windows_agree():
    n, m, rows, cols = 2, 4, 10, 64
    _, values, indices = _packed(rows, cols, n, m, 11)
    x1 = nm_synth.normal((5, cols), 1.0, 12, torch.float32)
    x2 = nm_synth.normal((5, cols), 1.0, 13, torch.float32)
    y1 = oracle.sparse_matmul(values, indices, x1, n, m)
    y2 = oracle.sparse_matmul(values, indices, x2, n, m)
    y3 = oracle.sparse_matmul(values, indices, x1 + 2 * x2, n, m)
    np.testing.assert_allclose(y3, y1 + 2 * y2, rtol=1e-6, atol=1e-6)
    win = oracle.sparse_matmul(values[3:8], indices[3:8], x1, n, m, rows=rows, row_begin=3)
    np.testing.assert_array_equal(win, y1[:, 3:8])
