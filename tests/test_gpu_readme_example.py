"""The usage example of README.md, run as written: its python block is executed on the GPU, then
its results are checked against what the example claims.
  * the loop trains: the logits received gradients and moved;
  * the packed form is the hard mask of the final logits: unpacking it keeps, in every group of
    four, the two weights of the first-argmax candidate (the candidate table of the library) and
    +0.0 elsewhere;
  * the product equals x times the transpose of that unpacked weight, computed by torch in fp32
    (within the fp32 accumulation bound of a 4096-term sum of bf16 products)."""
import os
import re
import sys

import pytest
import torch

import semi_structured_sparsity_amd as S

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README.md holds one python example"
    return blocks[0]


def test_readme_example_runs_and_its_outputs_hold():
    print("readme example", flush=True)
    sys.stdout.flush()
    env = {}
    exec(compile(_example(), "README.md", "exec"), env)
    torch.cuda.synchronize()
    w, logits, x, values, indices, y = (env[k] for k in ("w", "logits", "x", "values", "indices", "y"))
    prior = S.nm_prior_init(w, 2, 4, alpha=3.0)
    assert logits.grad is not None and torch.isfinite(logits.grad).all()
    assert not torch.equal(logits.detach(), prior)

    rows, cols = w.shape
    dense = S.nm_unpack(values, indices, cols, 2, 4)
    table = torch.tensor(S.candidate_table(2, 4), dtype=torch.int64, device=w.device)  # [K] bit patterns
    best = torch.argmax(logits.detach(), dim=-1)                                   # first maximal index
    bits = table[best]                                                              # [rows, cols/4]
    keep = torch.stack([(bits >> j) & 1 for j in range(4)], dim=-1).reshape(rows, cols).bool()
    want = torch.where(keep, w, torch.zeros_like(w))
    assert torch.equal(dense.view(torch.int16), want.view(torch.int16))

    ref = x.float() @ want.float().t()
    bound = 2 * 4096 * 2.0 ** -24 * (x.float().abs() @ want.float().abs().t()) + 1e-30  # both fp32 sums
    assert ((y.float() - ref).abs() <= bound + ref.abs() * 2.0 ** -8).all()  # y is bf16: half an ulp
