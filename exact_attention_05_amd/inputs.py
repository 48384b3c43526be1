"""Seeded synthetic inputs, shared by the GPU path's callers and the oracle tests.

This module holds none of the attention arithmetic: it only draws normal
samples and rounds them to the storage dtype.

Recipe (the same for every tensor):

* tensor ``name`` of head (b, h) is drawn from its own stream
  ``numpy.random.default_rng([seed, TENSOR_IDS[name], b, h])`` as
  ``standard_normal((rows, d), dtype=float32)``, multiplied by
  ``input_scale`` (0.5 for the long causal workload; a power of two, so the
  product is exact);
* it is rounded to the storage dtype by torch (round-to-nearest-even for
  bf16).

One stream per head lets a test regenerate any single head of a very large
tensor on the CPU, and lets the full tensor be drawn by a thread pool.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def head_normal(seed, name, b, h, rows, d, input_scale=1.0):
    """fp32 samples of head (b, h) of tensor ``name``: [rows, d]."""
    rng = np.random.default_rng([int(seed), TENSOR_IDS[name], int(b), int(h)])
    x = rng.standard_normal((rows, d), dtype=np.float32)
    if input_scale != 1.0:
        x *= np.float32(input_scale)
    return x


def make_head(seed, name, b, h, rows, d, dtype, input_scale=1.0):
    """Head (b, h) of ``make_tensor(seed, name, ...)`` as a CPU tensor [rows, d]."""
    return torch.from_numpy(head_normal(seed, name, b, h, rows, d, input_scale)).to(dtype)


def make_tensor(seed, name, B, H, rows, d, dtype, input_scale=1.0, device="cpu"):
    """A [B, H, rows, d] tensor in ``dtype`` following the recipe above.

    With ``device`` other than "cpu" the tensor is assembled head by head on
    the host and copied over, so host memory stays at a few heads.
    """
    out = torch.empty((B, H, rows, d), dtype=dtype, device=device)

    def fill(bh):
        b, h = divmod(bh, H)
        return bh, make_head(seed, name, b, h, rows, d, dtype, input_scale)

    with ThreadPoolExecutor(_threads()) as ex:
        for bh, t in ex.map(fill, range(B * H)):
            b, h = divmod(bh, H)
            out[b, h].copy_(t)
    return out


def widen(t):
    """Exact float64 copy of a CPU or device tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


def worked_example_qkv(d, dtype, rows=4):
    """Inputs whose scores with scale 1 are the 4-token example's blocks.

    Rows 0 and 1 of Q are [10, 20, 30, 5] and [10, 10, 5, 5] followed by zeros;
    rows 2 and 3 repeat them.  K = V = [I_4 | 0], so S = Q K^T has
    S_11 = [[10, 20], [10, 10]] and S_12 = [[30, 5], [5, 5]] for the first two
    query rows, and O rows equal the probability rows.  Every value is exact
    in bf16.  Returns CPU tensors [1, 1, rows, d].
    """
    q = torch.zeros((1, 1, rows, d), dtype=torch.float32)
    base = torch.tensor([[10.0, 20.0, 30.0, 5.0], [10.0, 10.0, 5.0, 5.0]])
    for r in range(rows):
        q[0, 0, r, :4] = base[r % 2]
    k = torch.zeros((1, 1, 4, d), dtype=torch.float32)
    k[0, 0, :, :4] = torch.eye(4)
    return q.to(dtype), k.to(dtype), k.clone().to(dtype)
