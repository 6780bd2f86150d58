"""Seeded synthetic inputs for the N:M mask layer: weights, logits and upstream gradients.

This module is shared by the tests, the benchmark and the smoke check.  It generates inputs
only; it contains none of the method's arithmetic (no noise of the method, softmax, masking,
packing or magnitude prior) and imports neither the HIP binding nor the oracle.  Every tensor
comes from a torch generator seeded explicitly.

Shapes follow the model families the MaskLLM project page evaluates (LLaMA-2 7B, Nemotron-4
15B).  Trained checkpoints are not available, so weights are Gaussian stand-ins with the
standard deviations below.  Prior-initialised logits (MaskLLM project page, Table 2 caption)
are assembled here from a prior candidate index that the caller computes: the tests take it
from the oracle, the benchmark from the library's own prior kernel.
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


def small_integers(shape, bound, seed, dtype=torch.bfloat16, device="cpu"):
    """Integers drawn uniformly from [-bound, bound], in `dtype` (exact in bf16 for bound <= 256):
    inputs whose products and partial sums are exact in fp32."""
    t = torch.randint(-bound, bound + 1, shape, generator=_gen(seed, device), device=device)
    return t.to(dtype)


def num_candidates(n, m):
    return len(list(itertools.combinations(range(m), n)))


PRIOR_ALPHA = 3.0       # logit of the prior candidate
PRIOR_NOISE_STD = 0.1   # N(0, 0.1) added to every logit


def prior_logits(prior_idx, K, seed, alpha=PRIOR_ALPHA, noise_std=PRIOR_NOISE_STD):
    """fp32 logits [rows, cols/m, K] on prior_idx's device: N(0, noise_std^2) everywhere plus
    alpha on the prior candidate prior_idx [rows, cols/m] (computed by the caller)."""
    idx = prior_idx.long()
    L = normal(tuple(idx.shape) + (K,), noise_std, seed, device=idx.device)
    L.scatter_add_(-1, idx.unsqueeze(-1), torch.full(tuple(idx.shape) + (1,), alpha, device=idx.device))
    return L


def gaussian_logits(rows, cols, n, m, seed, std=1.0, device="cpu"):
    return normal((rows, cols // m, num_candidates(n, m)), std, seed, device=device)


def input_seed(config, layer, matrix):
    """Seed of one matrix's inputs: 1000*config + 10*layer + matrix."""
    return 1000 * config + 10 * layer + matrix


def matrix_inputs(rows, cols, n, m, wtype, w_std, seed, logits="gaussian", with_grad=True,
                  device="cpu", prior=None):
    """(w, logits, grad) for one weight matrix; grad ~ N(0,1) in the weight type.  With
    logits="prior", `prior(w, n, m)` must return the prior candidate index of every group."""
    w = normal((rows, cols), w_std, 3 * seed + 0, wtype, device)
    if logits == "prior":
        if prior is None:
            raise ValueError("prior logits need the caller's prior(w, n, m)")
        L = prior_logits(prior(w, n, m).to(w.device), num_candidates(n, m), 3 * seed + 1)
    else:
        L = gaussian_logits(rows, cols, n, m, 3 * seed + 1, device=device)
    G = normal((rows, cols), 1.0, 3 * seed + 2, wtype, device) if with_grad else None
    return w, L, G
