"""Seeded synthetic inputs for the N:M mask layer: weights, logits and upstream gradients.

This module is shared by the tests, the benchmark and the smoke check.  It generates inputs
only; it contains none of the layer's arithmetic (no noise, softmax, masking or packing) and
imports neither the HIP binding nor the oracle.  Every tensor comes from a torch CPU generator
seeded explicitly, so the same call gives the same bits on any host.

Shapes follow the model families the MaskLLM project page evaluates (LLaMA-2 7B, Nemotron-4
15B).  Trained checkpoints are not available, so weights are Gaussian stand-ins with the
standard deviations below.  The magnitude prior follows the magnitude-pruning rule of the
"Accelerating Sparse Deep Neural Networks" page (section 4.1: keep the largest magnitudes of
each group), used as the prior mask that initialises the logits (MaskLLM project page,
Table 2 caption).
"""
import itertools

import torch

# (name, rows, cols) of the linear weights of one decoder layer, PyTorch [out, in] layout.
LLAMA2_7B_LAYER = [
    ("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
    ("down_proj", 4096, 11008),
]
# Hidden 6144, FFN 24576; no gate projection and full-width k/v (the only sizes known).
NEMOTRON_15B_LAYER = [
    ("q_proj", 6144, 6144), ("k_proj", 6144, 6144), ("v_proj", 6144, 6144),
    ("o_proj", 6144, 6144), ("up_proj", 24576, 6144), ("down_proj", 6144, 24576),
]
LAYERS = 32


def layer_weights(layer):
    return sum(r * c for _, r, c in layer)


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, dtype=torch.float32, device="cpu"):
    """N(0, std^2) samples (std is the standard deviation), rounded to `dtype`.  The same seed
    gives different values on different device types (each has its own generator)."""
    t = torch.randn(shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def num_candidates(n, m):
    return len(list(itertools.combinations(range(m), n)))


def magnitude_prior_index(w, n, m):
    """Index, in lexicographic candidate order, of the mask that keeps the n largest |w| of
    each group of m consecutive weights along the last dimension; ties keep the lower
    position.  Returns int64 [rows, cols/m]."""
    rows, cols = w.shape
    a = w.float().abs().reshape(rows, cols // m, m)
    # stable sort of -|w|: equal magnitudes keep their original (lower-first) order
    order = torch.sort(-a, dim=-1, stable=True).indices[..., :n]
    code = (torch.ones_like(order) << order).sum(-1)
    lut = torch.full((1 << m,), -1, dtype=torch.int64, device=w.device)
    for k, pos in enumerate(itertools.combinations(range(m), n)):
        lut[sum(1 << p for p in pos)] = k
    return lut[code]


def prior_logits(w, n, m, seed, alpha=3.0, noise_std=0.1):
    """fp32 logits [rows, cols/m, K] on w's device: alpha on the magnitude-prior candidate,
    0 elsewhere, plus N(0, noise_std^2)."""
    rows, cols = w.shape
    K = num_candidates(n, m)
    idx = magnitude_prior_index(w, n, m)
    L = normal((rows, cols // m, K), noise_std, seed, device=w.device)
    L.scatter_add_(-1, idx.unsqueeze(-1), torch.full(idx.shape + (1,), alpha, device=w.device))
    return L


def gaussian_logits(rows, cols, n, m, seed, std=1.0, device="cpu"):
    return normal((rows, cols // m, num_candidates(n, m)), std, seed, device=device)


def input_seed(config, layer, matrix):
    """Seed of one matrix's inputs: 1000*config + 10*layer + matrix."""
    return 1000 * config + 10 * layer + matrix


def matrix_inputs(rows, cols, n, m, wtype, w_std, seed, logits="gaussian", with_grad=True,
                  device="cpu"):
    """(w, logits, grad) for one weight matrix; grad ~ N(0,1) in the weight type."""
    w = normal((rows, cols), w_std, 3 * seed + 0, wtype, device)
    if logits == "prior":
        L = prior_logits(w, n, m, 3 * seed + 1)
    else:
        L = gaussian_logits(rows, cols, n, m, 3 * seed + 1, device=device)
    G = normal((rows, cols), 1.0, 3 * seed + 2, wtype, device) if with_grad else None
    return w, L, G
