"""Prior candidate indices for prior-initialised test inputs, computed by the oracle (the input
generator itself holds none of the method's arithmetic)."""
import numpy as np
import torch

import oracle


def oracle_prior(w, n, m):
    """int64 [rows, cols/m] on the CPU: the oracle's magnitude-prior candidate of every group."""
    _, idx = oracle.prior_init(w.detach().cpu(), n, m)
    return torch.from_numpy(idx.astype(np.int64))
