"""ctypes front end of the CPU oracle (oracle/nm_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the package smoke check and the CPU-baseline leg of
bench.py may import this package.  It shares no code with semi_structured_sparsity_amd and
never imports it.  Arrays are numpy arrays (or CPU torch tensors, converted without copying);
bf16 data travels as its raw uint16 bit patterns.  Every floating-point result is binary64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1  # weight element types, as in nm_oracle.h

_lib = None


class _Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("n", ctypes.c_int32),
                ("m", ctypes.c_int32), ("wtype", ctypes.c_int32)]


def lib():
    """Load (building first if needed) the oracle library."""
    global _lib
    if _lib is None:
        path = os.environ.get("NM_ORACLE_LIB")  # a test may point at a deliberately broken copy
        if path is None:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, u64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        sig = {
            "ref_num_candidates": (i32, [i32, i32]),
            "ref_candidate_bits": (i32, [i32, i32, P]),
            "ref_philox4x32": (None, [P, P, i32, P]),
            "ref_noise_word": (ctypes.c_uint32, [u64, u64, u64]),
            "ref_noise_words": (None, [u64, u64, u64, i64, P]),
            "ref_uniform": (dbl, [ctypes.c_uint32]),
            "ref_gumbel": (dbl, [ctypes.c_uint32]),
            "ref_gumbel_many": (None, [P, i64, P]),
            "ref_soft_mask": (i32, [P, dbl, dbl, u64, u64, i64, i64, P, P, i32]),
            "ref_forward": (i32, [P, dbl, dbl, u64, u64, i64, i64, P, P, P, i32]),
            "ref_backward": (i32, [P, dbl, dbl, u64, u64, i64, i64, P, P, P, P, i32]),
            "ref_backward_wreg": (i32, [P, dbl, dbl, u64, u64, dbl, i64, i64, P, P, P, P, i32]),
            "ref_probs": (i32, [P, dbl, dbl, u64, u64, i64, i64, P, P, i32]),
            "ref_index_words_per_row": (i64, [P]),
            "ref_harden": (i32, [P, i64, i64, P, P, i32]),
            "ref_pack": (i32, [P, i64, i64, P, P, P, P, P, i32]),
            "ref_unpack": (i32, [P, i64, i64, P, P, P, i32]),
            "ref_threads_used": (i32, [i32]),
            "ref_prior_init": (i32, [P, i64, i64, P, ctypes.c_float, P, P, i32]),
            "ref_monitor": (i32, [P, dbl, dbl, u64, u64, i64, i64, P, P, P, P, P, i32]),
            "ref_sparse_matmul": (i32, [P, i64, i64, P, P, P, i32, i64, P, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------------------------------------
# array plumbing

def _np(x):
    """numpy view of an array-like; bf16 torch tensors become their uint16 bit patterns."""
    if isinstance(x, np.ndarray):
        return x
    if hasattr(x, "detach"):  # torch tensor (CPU)
        import torch
        t = x.detach()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
            return t.numpy().view(np.uint16)
        return t.numpy()
    return np.asarray(x)


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _wtype_of(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"weights must be float32 or bf16 bits (uint16), got {a.dtype}")


def _contig(a, dtype=None):
    a = _np(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _unwritten(shape, dtype):
    """Output buffer whose every byte is 0xFF (NaN for floats), so that an element the oracle
    forgets to write cannot pass for a correct zero."""
    out = np.empty(shape, dtype)
    out.view(np.uint8)[...] = 0xFF
    return out


def _shape(rows, cols, n, m, wtype):
    return _Shape(rows, cols, n, m, wtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments of {what}")


# ---------------------------------------------------------------------------------------------
# candidates and noise

def num_candidates(n, m):
    return lib().ref_num_candidates(n, m)


def candidate_bits(n, m):
    """uint8 [K]: bit j of entry k is set iff candidate k keeps position j (lexicographic)."""
    K = num_candidates(n, m)
    if K < 0:
        raise ValueError(f"unsupported n:m = {n}:{m}")
    out = np.zeros(K, np.uint8)
    _check(lib().ref_candidate_bits(n, m, _ptr(out)), "candidate_bits")
    return out


def candidate_matrix(n, m):
    """float64 [K, m] 0/1 matrix of the candidates."""
    bits = candidate_bits(n, m)
    return ((bits[:, None] >> np.arange(m)[None, :]) & 1).astype(np.float64)


def philox4x32(ctr, key, rounds=10):
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().ref_philox4x32(_ptr(c), _ptr(k), rounds, _ptr(out))
    return out


def noise_words(seed, offset, first, count):
    out = np.zeros(count, np.uint32)
    lib().ref_noise_words(seed, offset, first, count, _ptr(out))
    return out


def uniform(x):
    return lib().ref_uniform(int(x))


def gumbel(x):
    """float64 Gumbel samples of uint32 words (vectorised)."""
    x = np.ascontiguousarray(x, np.uint32)
    out = np.zeros(x.shape, np.float64)
    lib().ref_gumbel_many(_ptr(x), x.size, _ptr(out))
    return out


def threads_used(nthreads=0):
    return lib().ref_threads_used(nthreads)


# ---------------------------------------------------------------------------------------------
# the layer (row windows: arrays hold rows [row_begin, row_end) of a rows x cols matrix)

def _window(arr_rows, row_begin, rows):
    row_end = row_begin + arr_rows
    if row_begin < 0 or row_end > rows:
        raise ValueError("row window outside the matrix")
    return row_end


def soft_mask(logits, n, m, kappa, tau, seed, offset, rows=None, row_begin=0, nthreads=0):
    """float64 soft mask [window_rows, cols] from fp32 logits [window_rows, cols/m, K]."""
    L = _contig(logits, np.float32)
    wr, gpr, K = L.shape
    rows = wr if rows is None else rows
    cols = gpr * m
    out = _unwritten((wr, cols), np.float64)
    s = _shape(rows, cols, n, m, F32)
    rc = lib().ref_soft_mask(ctypes.byref(s), kappa, tau, seed, offset, row_begin,
                             _window(wr, row_begin, rows), _ptr(L), _ptr(out), nthreads)
    _check(rc, "soft_mask")
    return out


def probs(logits, n, m, kappa, tau, seed, offset, rows=None, row_begin=0, nthreads=0):
    """float64 sampled probabilities y [window_rows, cols/m, K]."""
    L = _contig(logits, np.float32)
    wr, gpr, K = L.shape
    rows = wr if rows is None else rows
    out = _unwritten(L.shape, np.float64)
    s = _shape(rows, gpr * m, n, m, F32)
    rc = lib().ref_probs(ctypes.byref(s), kappa, tau, seed, offset, row_begin,
                         _window(wr, row_begin, rows), _ptr(L), _ptr(out), nthreads)
    _check(rc, "probs")
    return out


def forward(w, logits, n, m, kappa, tau, seed, offset, rows=None, row_begin=0, nthreads=0):
    """float64 masked weights [window_rows, cols] (not rounded to the weight type)."""
    W = _contig(w)
    L = _contig(logits, np.float32)
    wr, cols = W.shape
    rows = wr if rows is None else rows
    out = _unwritten((wr, cols), np.float64)
    s = _shape(rows, cols, n, m, _wtype_of(W))
    rc = lib().ref_forward(ctypes.byref(s), kappa, tau, seed, offset, row_begin,
                           _window(wr, row_begin, rows), _ptr(W), _ptr(L), _ptr(out), nthreads)
    _check(rc, "forward")
    return out


def backward(w, logits, grad, n, m, kappa, tau, seed, offset, rows=None, row_begin=0,
             nthreads=0):
    """float64 logit gradient [window_rows, cols/m, K]."""
    W = _contig(w)
    L = _contig(logits, np.float32)
    G = _contig(grad)
    if G.dtype != W.dtype or G.shape != W.shape:
        raise TypeError("grad must match w in shape and type")
    wr, cols = W.shape
    rows = wr if rows is None else rows
    out = _unwritten(L.shape, np.float64)
    s = _shape(rows, cols, n, m, _wtype_of(W))
    rc = lib().ref_backward(ctypes.byref(s), kappa, tau, seed, offset, row_begin,
                            _window(wr, row_begin, rows), _ptr(W), _ptr(L), _ptr(G), _ptr(out),
                            nthreads)
    _check(rc, "backward")
    return out


def backward_wreg(w, logits, grad, n, m, kappa, tau, seed, offset, lam, rows=None, row_begin=0,
                  nthreads=0):
    """float64 logit gradient [window_rows, cols/m, K] of the task loss (upstream grad, or None
    for none) plus lam * sum (w * soft_mask)^2 (MaskLLM project page, Table 3: weight
    regularisation; the squared norm of the masked weights is a reading, the page gives no
    formula)."""
    W = _contig(w)
    L = _contig(logits, np.float32)
    G = None
    if grad is not None:
        G = _contig(grad)
        if G.dtype != W.dtype or G.shape != W.shape:
            raise TypeError("grad must match w in shape and type")
    wr, cols = W.shape
    rows = wr if rows is None else rows
    out = _unwritten(L.shape, np.float64)
    s = _shape(rows, cols, n, m, _wtype_of(W))
    rc = lib().ref_backward_wreg(ctypes.byref(s), kappa, tau, seed, offset, float(lam), row_begin,
                                 _window(wr, row_begin, rows), _ptr(W), _ptr(L),
                                 None if G is None else _ptr(G), _ptr(out), nthreads)
    _check(rc, "backward_wreg")
    return out


def index_words_per_row(cols, n, m):
    s = _shape(1, cols, n, m, F32)
    return lib().ref_index_words_per_row(ctypes.byref(s))


def harden(logits, n, m, nthreads=0):
    """uint8 [rows, cols/m]: index of the first largest logit of each group."""
    L = _contig(logits, np.float32)
    wr, gpr, K = L.shape
    out = _unwritten((wr, gpr), np.uint8)
    s = _shape(wr, gpr * m, n, m, F32)
    _check(lib().ref_harden(ctypes.byref(s), 0, wr, _ptr(L), _ptr(out), nthreads), "harden")
    return out


def pack(w, logits, n, m, nthreads=0):
    """(values [rows, cols*n/m] same dtype as w, indices uint32 [rows, words], hard uint8)."""
    W = _contig(w)
    L = _contig(logits, np.float32)
    wr, cols = W.shape
    s = _shape(wr, cols, n, m, _wtype_of(W))
    wpr = lib().ref_index_words_per_row(ctypes.byref(s))
    values = _unwritten((wr, cols // m * n), W.dtype)
    idx = _unwritten((wr, wpr), np.uint32)
    hard = _unwritten((wr, cols // m), np.uint8)
    rc = lib().ref_pack(ctypes.byref(s), 0, wr, _ptr(W), _ptr(L), _ptr(values), _ptr(idx),
                        _ptr(hard), nthreads)
    _check(rc, "pack")
    return values, idx, hard


def unpack(values, indices, cols, n, m, nthreads=0):
    """dense [rows, cols] (dtype of values)."""
    V = _contig(values)
    I = _contig(indices, np.uint32)
    wr = V.shape[0]
    s = _shape(wr, cols, n, m, _wtype_of(V))
    if I.shape != (wr, lib().ref_index_words_per_row(ctypes.byref(s))):
        raise ValueError("indices shape does not match")
    out = _unwritten((wr, cols), V.dtype)
    rc = lib().ref_unpack(ctypes.byref(s), 0, wr, _ptr(V), _ptr(I), _ptr(out), nthreads)
    _check(rc, "unpack")
    return out


def prior_init(w, n, m, alpha=3.0, rows=None, row_begin=0, nthreads=0):
    """(logits fp32 [window_rows, cols/m, K], prior index uint8 [window_rows, cols/m])."""
    W = _contig(w)
    wr, cols = W.shape
    rows = wr if rows is None else rows
    K = num_candidates(n, m)
    logits = _unwritten((wr, cols // m, K), np.float32)
    idx = _unwritten((wr, cols // m), np.uint8)
    s = _shape(rows, cols, n, m, _wtype_of(W))
    rc = lib().ref_prior_init(ctypes.byref(s), row_begin, _window(wr, row_begin, rows), _ptr(W), alpha,
                              _ptr(logits), _ptr(idx), nthreads)
    _check(rc, "prior_init")
    return logits, idx


def monitor(logits, n, m, kappa, tau, seed, offset, prev_sample=None, rows=None, row_begin=0,
            nthreads=0):
    """Per group of the window: (max probability of softmax(kappa*l) float64, sampled candidate
    uint8, L1 distance to prev_sample uint8 or None) -- all [window_rows, cols/m]."""
    L = _contig(logits, np.float32)
    wr, gpr, K = L.shape
    rows = wr if rows is None else rows
    maxp = _unwritten((wr, gpr), np.float64)
    samp = _unwritten((wr, gpr), np.uint8)
    prev = None if prev_sample is None else _contig(prev_sample, np.uint8)
    if prev is not None and prev.shape != (wr, gpr):
        raise ValueError("prev_sample must be [window_rows, cols/m]")
    l1 = None if prev is None else _unwritten((wr, gpr), np.uint8)
    s = _shape(rows, gpr * m, n, m, F32)
    rc = lib().ref_monitor(ctypes.byref(s), kappa, tau, seed, offset, row_begin,
                           _window(wr, row_begin, rows), _ptr(L), None if prev is None else _ptr(prev),
                           _ptr(maxp), _ptr(samp), None if l1 is None else _ptr(l1), nthreads)
    _check(rc, "monitor")
    return maxp, samp, l1


def sparse_matmul(values, indices, x, n, m, rows=None, row_begin=0, nthreads=0):
    """float64 Y [tokens, window_rows] = X times the transpose of the unpacked weights, from the
    packed form (values [window_rows, cols*n/m], indices [window_rows, words]) of W rows
    row_begin .. row_begin + window_rows - 1.  x: [tokens, cols] float32 or bf16."""
    V = _contig(values)
    I = _contig(indices, np.uint32)
    X = _contig(x)
    wr = V.shape[0]
    rows = wr if rows is None else rows
    tokens, cols = X.shape
    if V.shape[1] != cols // m * n:
        raise ValueError("values do not match x's columns")
    y = _unwritten((tokens, wr), np.float64)
    s = _shape(rows, cols, n, m, _wtype_of(V))
    rc = lib().ref_sparse_matmul(ctypes.byref(s), row_begin, _window(wr, row_begin, rows), _ptr(V), _ptr(I),
                                 _ptr(X), _wtype_of(X), tokens, _ptr(y), nthreads)
    _check(rc, "sparse_matmul")
    return y
