"""Learnable N:M semi-structured sparsity on MI355X: Python binding of libnm_mask.so.

The binding only marshals arguments: every step of the layer runs in the HIP kernels of
libnm_mask.so (include/nm_mask.h documents the contract).  PyTorch provides device memory and
the current stream.  Importing the package does not touch the GPU; the first call loads the
library and fails loudly if it has not been built (python -m semi_structured_sparsity_amd.build)
or if a tensor is not on a ROCm device.

Entry points, named as in the C ABI:
    nm_mask_forward(w, logits, n, m, kappa, tau, seed, offset)        -> w_masked
    nm_mask_backward(w, logits, grad, n, m, kappa, tau, seed, offset) -> grad_logits
    nm_mask_backward_wreg(w, logits, grad_or_None, n, m, kappa, tau, seed, offset, lam)
                                                                      -> grad_logits
    nm_mask_harden_pack(w, logits, n, m, with_hard=False)             -> values, indices[, hard]
    nm_mask_forward_pack(w, logits, n, m, kappa, tau, seed, offset, with_hard=False)
                                                                      -> w_masked, values, indices[, hard]
    nm_unpack(values, indices, cols, n, m)                            -> w_dense
    nm_prior_init(w, n, m, alpha, with_idx=False)                     -> logits[, prior_idx]
    nm_mask_forward_monitor(w, logits, n, m, kappa, tau, seed, offset, prev_sample=None)
                                                                      -> w_masked, sample, stats
    nm_mask_forward_monitor_static(...)                               the same, with no workspace
and `mask(...)`, the autograd function whose backward is nm_mask_backward, or
nm_mask_backward_wreg when a weight-regulariser strength is given (the weights are frozen and get
no gradient).
"""
import ctypes
import os

import torch

from . import build as _build

NM_OK, NM_EINVAL, NM_EALIGN, NM_EUNSUPPORTED, NM_EHIP, NM_ESCRATCH = range(6)
MONITOR_SCRATCH_BYTES = 1 << 16  # NM_MONITOR_SCRATCH_BYTES
NM_F32, NM_BF16 = 0, 1

_lib = None


class NMError(RuntimeError):
    """A non-zero nm_status from the library."""

    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {lib().nm_status_str(status).decode()} (status {status})")


class _Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("n", ctypes.c_int32),
                ("m", ctypes.c_int32), ("wtype", ctypes.c_int32)]


class _Sample(ctypes.Structure):
    _fields_ = [("kappa", ctypes.c_float), ("tau", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "nm_mask_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "nm_mask_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "nm_mask_backward_wreg": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, _P, _P, _P, _P]),
    "nm_mask_forward_pack": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nm_mask_forward_offset_dev": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "nm_mask_backward_offset_dev": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "nm_mask_harden_pack": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "nm_unpack": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "nm_prior_init": (ctypes.c_int, [_P, ctypes.c_float, _P, _P, _P, _P]),
    "nm_mask_forward_monitor": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int64, _P]),
    "nm_mask_forward_monitor_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nm_monitor_workspace_bytes": (ctypes.c_int64, [_P]),
    "nm_sparse_matmul": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_int32, _P]),
    "nm_sparse_matmul_ws": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_int32, _P, ctypes.c_int64, _P]),
    "nm_sparse_matmul_workspace_bytes": (ctypes.c_int64, [_P, ctypes.c_int64]),
    "nm_sparse_matmul_plan": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
    "nm_num_candidates": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32]),
    "nm_candidate_table": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P]),
    "nm_packed_value_elems": (ctypes.c_int64, [_P]),
    "nm_index_words_per_row": (ctypes.c_int64, [_P]),
    "nm_packed_index_words": (ctypes.c_int64, [_P]),
    "nm_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "nm_debug_noise": (ctypes.c_int, [_P, _P, _P, _P]),
    "nm_debug_gumbel_log2": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "nm_debug_copy": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "nm_debug_soft_mask": (ctypes.c_int, [_P, _P, _P, _P, _P]),
}
EXPORTS = tuple(_SIGNATURES)


def library_path():
    return os.environ.get("NM_MASK_LIB", _build.LIB)


def lib():
    """The loaded libnm_mask.so (never rebuilt here: build() does that explicitly)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m semi_structured_sparsity_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------------------------------------
# marshalling helpers

def _wtype(dtype):
    if dtype == torch.float32:
        return NM_F32
    if dtype == torch.bfloat16:
        return NM_BF16
    raise TypeError(f"weights must be float32 or bfloat16, got {dtype}")


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(rows, cols, n, m, wtype):
    return _Shape(int(rows), int(cols), int(n), int(m), int(wtype))


def _sample(kappa, tau, seed, offset):
    return _Sample(float(kappa), float(tau), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1))


def _check(status, what):
    if status != NM_OK:
        raise NMError(status, what)


def num_candidates(n, m):
    """K = C(m, n) for a supported n:m, else -1."""
    return lib().nm_num_candidates(n, m)


def candidate_table(n, m):
    """Host list of K bytes: bit j of entry k set iff candidate k keeps position j."""
    K = num_candidates(n, m)
    if K < 0:
        raise NMError(NM_EUNSUPPORTED, "nm_candidate_table")
    buf = (ctypes.c_uint8 * K)()
    _check(lib().nm_candidate_table(n, m, buf), "nm_candidate_table")
    return list(buf)


def index_words_per_row(cols, n, m):
    return lib().nm_index_words_per_row(ctypes.byref(_shape(1, cols, n, m, NM_F32)))


def _logit_shape(rows, cols, n, m):
    K = num_candidates(n, m)
    if K < 0:
        raise NMError(NM_EUNSUPPORTED, "n:m")
    return (rows, cols // m, K)


# ---------------------------------------------------------------------------------------------
# the four entry points of the layer

def _offset_dev(offset):
    """A one-element int64 device tensor holding the step offset (read when the kernels run)."""
    if offset.dtype != torch.int64 or offset.numel() != 1:
        raise TypeError("a device offset must be a one-element int64 tensor")
    return _dev(offset, "offset")


def nm_mask_forward(w, logits, n, m, kappa, tau, seed, offset, out=None):
    """Masked frozen weights w * m (MaskLLM project page, Fig. 3 caption).  `offset` is the
    step: an int, or a one-element int64 tensor on the device, read when the kernel runs
    (nm_mask_forward_offset_dev: a captured graph then samples each replay's step)."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    out = torch.empty_like(w) if out is None else out
    lshape = _logit_shape(rows, cols, n, m)
    if isinstance(offset, torch.Tensor):
        st = lib().nm_mask_forward_offset_dev(
            ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, 0)), _offset_dev(offset), _dev(w, "w"),
            _dev(logits, "logits", torch.float32, lshape), _dev(out, "out", w.dtype, w.shape), _stream(w.device))
        _check(st, "nm_mask_forward_offset_dev")
        return out
    st = lib().nm_mask_forward(ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)),
                               _dev(w, "w"), _dev(logits, "logits", torch.float32, lshape),
                               _dev(out, "out", w.dtype, w.shape), _stream(w.device))
    _check(st, "nm_mask_forward")
    return out


def monitor_workspace_bytes(rows, cols, n, m):
    return lib().nm_monitor_workspace_bytes(ctypes.byref(_shape(rows, cols, n, m, NM_F32)))


def nm_mask_forward_monitor(w, logits, n, m, kappa, tau, seed, offset, prev_sample=None, out=None,
                            workspace=None):
    """The forward plus the convergence monitors (MaskLLM project page, Fig. 5 caption).
    Returns (w_masked, sample uint8 [rows, cols/m], stats float64 [2] on the device) with
    stats = (sum of the largest probability of softmax(kappa*l), sum of the L1 distance between
    this step's sampled mask and prev_sample's) over all groups.  A `workspace` passed in must
    have been zero-filled before its first use (every call leaves it zero-filled again)."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    need = lib().nm_monitor_workspace_bytes(ctypes.byref(sh))
    if need < 0:
        raise NMError(NM_EINVAL, "nm_mask_forward_monitor")
    if out is None:
        out = (torch.empty_like(w), torch.empty((rows, cols // m), dtype=torch.uint8, device=w.device),
               torch.zeros(2, dtype=torch.float64, device=w.device))
    w_masked, sample, stats = out
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=w.device)  # zero before first use
    gshape = (rows, cols // m)
    st = lib().nm_mask_forward_monitor(
        ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)), _dev(w, "w"),
        _dev(logits, "logits", torch.float32, _logit_shape(rows, cols, n, m)),
        _dev(w_masked, "w_masked", w.dtype, w.shape),
        None if prev_sample is None else _dev(prev_sample, "prev_sample", torch.uint8, gshape),
        None if sample is None else _dev(sample, "sample", torch.uint8, gshape),
        _dev(stats, "stats", torch.float64, (2,)), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(w.device))
    _check(st, "nm_mask_forward_monitor")
    return w_masked, sample, stats


def nm_mask_forward_monitor_static(w, logits, n, m, kappa, tau, seed, offset, prev_sample=None, out=None):
    """nm_mask_forward_monitor without a workspace: the partial sums live in the library's fixed
    device array (NM_MONITOR_SCRATCH_BYTES per GPU), for callers that cannot allocate.  With
    `out` given, nothing is allocated here either.  Calls whose executions overlap on one GPU
    race on that array."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    if out is None:
        out = (torch.empty_like(w), torch.empty((rows, cols // m), dtype=torch.uint8, device=w.device),
               torch.zeros(2, dtype=torch.float64, device=w.device))
    w_masked, sample, stats = out
    gshape = (rows, cols // m)
    st = lib().nm_mask_forward_monitor_static(
        ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)), _dev(w, "w"),
        _dev(logits, "logits", torch.float32, _logit_shape(rows, cols, n, m)),
        _dev(w_masked, "w_masked", w.dtype, w.shape),
        None if prev_sample is None else _dev(prev_sample, "prev_sample", torch.uint8, gshape),
        None if sample is None else _dev(sample, "sample", torch.uint8, gshape),
        _dev(stats, "stats", torch.float64, (2,)), _stream(w.device))
    _check(st, "nm_mask_forward_monitor_static")
    return w_masked, sample, stats


def nm_mask_backward(w, logits, grad, n, m, kappa, tau, seed, offset, out=None):
    """Gradient of the loss with respect to the logits (overwrites `out` if given).  `offset` as
    in nm_mask_forward (an int, or a one-element int64 device tensor)."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    lshape = _logit_shape(rows, cols, n, m)
    out = torch.empty(lshape, dtype=torch.float32, device=w.device) if out is None else out
    if isinstance(offset, torch.Tensor):
        st = lib().nm_mask_backward_offset_dev(
            ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, 0)), _offset_dev(offset), _dev(w, "w"),
            _dev(logits, "logits", torch.float32, lshape), _dev(grad, "grad", w.dtype, w.shape),
            _dev(out, "out", torch.float32, lshape), _stream(w.device))
        _check(st, "nm_mask_backward_offset_dev")
        return out
    st = lib().nm_mask_backward(ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)),
                                _dev(w, "w"), _dev(logits, "logits", torch.float32, lshape),
                                _dev(grad, "grad", w.dtype, w.shape),
                                _dev(out, "out", torch.float32, lshape), _stream(w.device))
    _check(st, "nm_mask_backward")
    return out


def nm_mask_backward_wreg(w, logits, grad, n, m, kappa, tau, seed, offset, lam, out=None):
    """Logit gradient of the task loss (upstream `grad`, or None for none) plus the weight
    regulariser lam * sum (w * m)^2 (MaskLLM project page, Table 3; the squared norm of the
    masked weights is the reading taken, the page gives no formula)."""
    if isinstance(offset, torch.Tensor):
        raise TypeError("nm_mask_backward_wreg takes the step offset as an int")
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    lshape = _logit_shape(rows, cols, n, m)
    out = torch.empty(lshape, dtype=torch.float32, device=w.device) if out is None else out
    st = lib().nm_mask_backward_wreg(
        ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)), float(lam), _dev(w, "w"),
        _dev(logits, "logits", torch.float32, lshape),
        None if grad is None else _dev(grad, "grad", w.dtype, w.shape),
        _dev(out, "out", torch.float32, lshape), _stream(w.device))
    _check(st, "nm_mask_backward_wreg")
    return out


def nm_mask_harden_pack(w, logits, n, m, with_hard=False, out=None):
    """Hard argmax mask packed as (values, indices[, hard]) ("Accelerating Sparse Deep Neural
    Networks" summary page, section 3.1)."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    wpr = lib().nm_index_words_per_row(ctypes.byref(sh))
    if wpr < 0:
        raise NMError(NM_EINVAL, "nm_mask_harden_pack")
    if out is None:
        values = torch.empty((rows, cols // m * n), dtype=w.dtype, device=w.device)
        indices = torch.empty((rows, wpr), dtype=torch.int32, device=w.device)
        hard = torch.empty((rows, cols // m), dtype=torch.uint8, device=w.device) if with_hard else None
    else:
        values, indices, hard = out
    st = lib().nm_mask_harden_pack(
        ctypes.byref(sh), _dev(w, "w"),
        _dev(logits, "logits", torch.float32, _logit_shape(rows, cols, n, m)),
        _dev(values, "values", w.dtype, (rows, cols // m * n)),
        _dev(indices, "indices", torch.int32, (rows, wpr)),
        None if hard is None else _dev(hard, "hard", torch.uint8, (rows, cols // m)),
        _stream(w.device))
    _check(st, "nm_mask_harden_pack")
    return (values, indices, hard) if with_hard else (values, indices)


def nm_mask_forward_pack(w, logits, n, m, kappa, tau, seed, offset, with_hard=False, out=None):
    """(w_masked, values, indices[, hard]): nm_mask_forward and nm_mask_harden_pack of the same
    inputs in one call (one pass over w and the logits for 2:4 when cols/4 is a multiple of 8)."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    wpr = index_words_per_row(cols, n, m)
    lshape = _logit_shape(rows, cols, n, m)
    if out is None:
        out = (torch.empty_like(w), torch.empty((rows, cols // m * n), dtype=w.dtype, device=w.device),
               torch.empty((rows, wpr), dtype=torch.int32, device=w.device),
               torch.empty((rows, cols // m), dtype=torch.uint8, device=w.device) if with_hard else None)
    w_masked, values, indices, hard = out
    st = lib().nm_mask_forward_pack(
        ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)), _dev(w, "w"),
        _dev(logits, "logits", torch.float32, lshape), _dev(w_masked, "w_masked", w.dtype, w.shape),
        _dev(values, "values", w.dtype, (rows, cols // m * n)), _dev(indices, "indices", torch.int32, (rows, wpr)),
        None if hard is None else _dev(hard, "hard", torch.uint8, (rows, cols // m)), _stream(w.device))
    _check(st, "nm_mask_forward_pack")
    return (w_masked, values, indices, hard) if hard is not None else (w_masked, values, indices)


def nm_unpack(values, indices, cols, n, m, out=None):
    """Dense weights with +0.0 at dropped positions."""
    rows = values.shape[0]
    sh = _shape(rows, cols, n, m, _wtype(values.dtype))
    wpr = lib().nm_index_words_per_row(ctypes.byref(sh))
    if wpr < 0:
        raise NMError(NM_EINVAL, "nm_unpack")
    out = torch.empty((rows, cols), dtype=values.dtype, device=values.device) if out is None else out
    st = lib().nm_unpack(ctypes.byref(sh), _dev(values, "values", None, (rows, cols // m * n)),
                         _dev(indices, "indices", torch.int32, (rows, wpr)),
                         _dev(out, "out", values.dtype, (rows, cols)), _stream(values.device))
    _check(st, "nm_unpack")
    return out


def nm_prior_init(w, n, m, alpha, with_idx=False, out=None):
    """Logits initialised from the magnitude prior: alpha on the candidate keeping the n largest
    |w| of each group, 0 elsewhere (MaskLLM project page, Table 2 caption; "Accelerating Sparse
    Deep Neural Networks" summary page, section 4.1).  Returns logits[, prior_idx uint8]."""
    rows, cols = w.shape
    sh = _shape(rows, cols, n, m, _wtype(w.dtype))
    lshape = _logit_shape(rows, cols, n, m)
    if out is None:
        logits = torch.empty(lshape, dtype=torch.float32, device=w.device)
        idx = torch.empty((rows, cols // m), dtype=torch.uint8, device=w.device) if with_idx else None
    else:
        logits, idx = out
    st = lib().nm_prior_init(ctypes.byref(sh), float(alpha), _dev(w, "w"),
                             _dev(logits, "logits", torch.float32, lshape),
                             None if idx is None else _dev(idx, "prior_idx", torch.uint8, (rows, cols // m)),
                             _stream(w.device))
    _check(st, "nm_prior_init")
    return (logits, idx) if with_idx else logits


# Workspace sizes of the product by (device, out, in, weight type, tokens): the plan depends
# only on these (and on the device's compute units), so the binding asks the library once.
_SPMM_NEED = {}


def _spmm_need(sh, device, tokens):
    key = (device.index, sh.rows, sh.cols, sh.wtype, tokens)
    need = _SPMM_NEED.get(key)
    if need is None:
        need = lib().nm_sparse_matmul_workspace_bytes(ctypes.byref(sh), tokens)
        if len(_SPMM_NEED) > 4096:
            _SPMM_NEED.clear()
        _SPMM_NEED[key] = need
    return need


def sparse_matmul_workspace_bytes(out, inn, tokens):
    """Workspace bytes nm_sparse_matmul needs for W [out, inn] and `tokens` tokens on the current
    device (0 when the product does not split its k range)."""
    return lib().nm_sparse_matmul_workspace_bytes(ctypes.byref(_shape(out, inn, 2, 4, NM_BF16)), int(tokens))


def sparse_matmul_plan(out, inn, tokens, split=True):
    """(tile, parts) nm_sparse_matmul runs W [out, inn] at `tokens` tokens with on the current
    device: tile 0 row streaming, 16 the 16-row kernel, 64/128/256 the tiles; parts of the k
    range (1 without split); (-1, 0) for an empty product."""
    tile, parts = ctypes.c_int32(), ctypes.c_int32()
    st = lib().nm_sparse_matmul_plan(ctypes.byref(_shape(out, inn, 2, 4, NM_BF16)), int(tokens), int(bool(split)),
                                     ctypes.byref(tile), ctypes.byref(parts))
    _check(st, "nm_sparse_matmul_plan")
    return tile.value, parts.value


def nm_sparse_matmul(values, indices, x, out_dtype=torch.bfloat16, out=None, workspace=None, split=True):
    """Y [tokens, out] = X [tokens, in] times the transpose of the 2:4 weights W [out, in] held in
    nm_mask_harden_pack's packed form (values [out, in/2] bf16, indices [out, in/32]), on the
    sparse matrix cores ("Accelerating Sparse Deep Neural Networks" summary page, 3.1-3.2).
    With `split`, mid-size batches split the k range over a workspace (nm_sparse_matmul_ws):
    `workspace`, a uint8 device tensor of at least sparse_matmul_workspace_bytes bytes, or one
    allocated here; split=False calls nm_sparse_matmul, which never splits."""
    rows, half = values.shape
    tokens, cols = x.shape
    if cols != 2 * half:
        raise ValueError(f"x has {cols} columns, the packed weights {2 * half}")
    sh = _shape(rows, cols, 2, 4, _wtype(values.dtype))
    ytype = _wtype(out_dtype)
    y = torch.empty((tokens, rows), dtype=out_dtype, device=x.device) if out is None else out
    if not split:
        st = lib().nm_sparse_matmul(ctypes.byref(sh), _dev(values, "values"),
                                    _dev(indices, "indices", torch.int32, (rows, cols // 32)),
                                    _dev(x, "x", torch.bfloat16), tokens,
                                    _dev(y, "y", out_dtype, (tokens, rows)), ytype, _stream(x.device))
        _check(st, "nm_sparse_matmul")
        return y
    need = _spmm_need(sh, x.device, tokens)
    if need < 0:
        raise NMError(NM_EUNSUPPORTED, "nm_sparse_matmul")
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws = None if need == 0 else _dev(workspace, "workspace", torch.uint8)
    st = lib().nm_sparse_matmul_ws(ctypes.byref(sh), _dev(values, "values"),
                                   _dev(indices, "indices", torch.int32, (rows, cols // 32)),
                                   _dev(x, "x", torch.bfloat16), tokens,
                                   _dev(y, "y", out_dtype, (tokens, rows)), ytype, ws,
                                   0 if workspace is None else workspace.numel(), _stream(x.device))
    _check(st, "nm_sparse_matmul")
    return y


# ---------------------------------------------------------------------------------------------
# diagnostics (same device functions as the kernels)

def nm_debug_noise(rows, cols, n, m, seed, offset, device="cuda"):
    """Raw Philox words [rows, cols/m, K] as int32 (bit patterns of the uint32 words)."""
    shape = _logit_shape(rows, cols, n, m)
    out = torch.empty(shape, dtype=torch.int32, device=device)
    sh = _shape(rows, cols, n, m, NM_F32)
    st = lib().nm_debug_noise(ctypes.byref(sh), ctypes.byref(_sample(1.0, 1.0, seed, offset)),
                              _dev(out, "out"), _stream(out.device))
    _check(st, "nm_debug_noise")
    return out


def nm_debug_gumbel_log2(words):
    """h = log2(-log2(u)) for int32 tensors holding uint32 noise words."""
    out = torch.empty(words.shape, dtype=torch.float32, device=words.device)
    st = lib().nm_debug_gumbel_log2(_dev(words, "words", torch.int32), _dev(out, "out"),
                                    words.numel(), _stream(words.device))
    _check(st, "nm_debug_gumbel_log2")
    return out


def nm_debug_copy(src, dst):
    """dst <- src with the path kernels' access pattern (both contiguous, same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    st = lib().nm_debug_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes, _stream(src.device))
    _check(st, "nm_debug_copy")
    return dst


def nm_debug_soft_mask(logits, n, m, kappa, tau, seed, offset):
    """fp32 soft mask [rows, cols] of a sample."""
    rows, gpr, K = logits.shape
    cols = gpr * m
    out = torch.empty((rows, cols), dtype=torch.float32, device=logits.device)
    sh = _shape(rows, cols, n, m, NM_F32)
    st = lib().nm_debug_soft_mask(ctypes.byref(sh), ctypes.byref(_sample(kappa, tau, seed, offset)),
                                  _dev(logits, "logits", torch.float32, _logit_shape(rows, cols, n, m)),
                                  _dev(out, "out"), _stream(logits.device))
    _check(st, "nm_debug_soft_mask")
    return out


# ---------------------------------------------------------------------------------------------
# autograd

class NMMask(torch.autograd.Function):
    """w_masked = w * softmask(logits); gradient to the logits only (frozen weights).  With
    wreg != 0 the gradient also carries the regulariser wreg * sum(w_masked^2), which the caller
    then leaves out of its own loss."""

    @staticmethod
    def forward(ctx, w, logits, n, m, kappa, tau, seed, offset, wreg=0.0):
        ctx.save_for_backward(w, logits)
        ctx.params = (n, m, kappa, tau, seed, offset, wreg)
        return nm_mask_forward(w, logits, n, m, kappa, tau, seed, offset)

    @staticmethod
    def backward(ctx, grad):
        w, logits = ctx.saved_tensors
        n, m, kappa, tau, seed, offset, wreg = ctx.params
        if wreg != 0.0:
            dl = nm_mask_backward_wreg(w, logits, grad.contiguous(), n, m, kappa, tau, seed, offset, wreg)
        else:
            dl = nm_mask_backward(w, logits, grad.contiguous(), n, m, kappa, tau, seed, offset)
        return None, dl, None, None, None, None, None, None, None


def mask(w, logits, n, m, kappa, tau, seed, offset, wreg=0.0):
    """Differentiable N:M mask layer; `offset` is the training step (fresh noise per step).
    `wreg` adds the gradient of wreg * sum(w_masked^2) in the backward (fused: no extra pass)."""
    return NMMask.apply(w, logits, n, m, kappa, tau, seed, offset, wreg)


def packed_bytes(rows, cols, n, m, elem_bytes):
    """Bytes of the compressed form: kept values plus index words."""
    return rows * cols // m * n * elem_bytes + rows * index_words_per_row(cols, n, m) * 4


__all__ = ["nm_mask_forward", "nm_mask_backward", "nm_mask_backward_wreg", "nm_mask_harden_pack",
           "nm_mask_forward_pack", "nm_unpack",
           "nm_prior_init", "nm_mask_forward_monitor", "monitor_workspace_bytes", "nm_debug_noise",
           "nm_debug_copy", "nm_sparse_matmul", "sparse_matmul_workspace_bytes", "sparse_matmul_plan",
           "nm_debug_gumbel_log2",
           "nm_debug_soft_mask", "mask", "NMMask",
           "num_candidates", "candidate_table", "index_words_per_row", "packed_bytes", "lib",
           "NMError", "EXPORTS", "library_path"]
