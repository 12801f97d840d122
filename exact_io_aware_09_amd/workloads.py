"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

Both the HIP path and the CPU oracle receive the tensors made here; nothing
in this module computes any part of attention.

Recipe: ``g = torch.Generator('cpu').manual_seed(seed)``; Q, K, V, dO are
drawn in that order as float32 N(0, 1) of shape [B, H, N, d], multiplied by
``mult`` (0.5 for the large head-dim shape; exact in binary), then rounded to
the compute dtype (round-to-nearest-even for bfloat16).  The oracle gets the
same rounded values upcast to float64.  The shapes are the pages' own
workloads: GPT-2-medium attention (B 64, H 16, N 1024, d 64) and the
memory-footprint shape (B 16, H 8, N 4096, d 64) measured on A100 in
"FlashAttention and GPU memory" sections 01, 09 and 10; the N = 65,536
long-sequence shape from the same section; and head dim 256 at long
sequence, where the third version's forward throughput is quoted (section
11); and a small-batch, few-head shape (B 1, H 8, N 4096, d 64) whose 256
query blocks alone leave most of the GPU idle, the case of the key-split forward
("Lecture 8", section 8.2).  Synthetic N(0, 1) data stands in for activations
because the pages time the operation itself, not a trained model.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    causal: bool
    scale: float
    seed: int
    mult: float = 1.0
    sampled: bool = False  # oracle checks sampled rows instead of full tensors
    description: str = field(default="", compare=False)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, torch.float32, False, 1.0 / 8.0, 0,
                     description="exact check, fp32, non-causal"),
    "gpt2_medium": Workload("gpt2_medium", 64, 16, 1024, 64, torch.bfloat16, True, 1.0 / 8.0, 1,
                            description="GPT-2-medium attention shape, bf16, causal"),
    "memory": Workload("memory", 16, 8, 4096, 64, torch.bfloat16, False, 1.0 / 8.0, 2,
                       description="memory-footprint shape, bf16, non-causal"),
    "long": Workload("long", 1, 8, 65536, 64, torch.bfloat16, True, 1.0 / 8.0, 3, sampled=True,
                     description="long sequence, bf16, causal, no N x N buffer"),
    "big_d": Workload("big_d", 2, 16, 16384, 256, torch.bfloat16, False, 1.0 / 16.0, 4, mult=0.5,
                      sampled=True, description="head dim 256, bf16 x0.5, non-causal"),
    # the split-KV forward's case: B*H*N/128 = 256 query blocks, one per CU,
    # a quarter of the workgroups the GPU holds at once
    "few_heads": Workload("few_heads", 1, 8, 4096, 64, torch.bfloat16, False, 1.0 / 8.0, 5,
                          sampled=True, description="small batch, few heads, bf16, non-causal"),
}


def make_inputs(shape, dtype, seed: int, mult: float = 1.0):
    """(Q, K, V, dO) on the CPU in ``dtype``, drawn from one seeded generator."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for _ in range(4):
        t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
        if mult != 1.0:
            t.mul_(mult)
        out.append(t.to(dtype))
    return tuple(out)


def workload_inputs(w: Workload):
    return make_inputs(w.shape, w.dtype, w.seed, w.mult)


def sample_rows(seed: int, b: int, h: int, H: int, N: int, count: int = 256, edges=(0, 1, 31, 32, 63, 64, 127, 128, 255, 256)):
    """Distinct query and key row indices for head (b, h), plus edge rows.

    ``numpy.random.default_rng(seed + 1000 + b*H + h)`` draws ``count``
    distinct query rows then ``count`` distinct key rows; the edge rows (and
    N-1) are appended to both.  Returns sorted int64 arrays.
    """
    rng = np.random.default_rng(int(seed) + 1000 + b * H + h)
    k = min(count, N)
    qi = rng.choice(N, size=k, replace=False)
    ki = rng.choice(N, size=k, replace=False)
    extra = [e for e in (*edges, N - 1) if 0 <= e < N]
    qi = np.unique(np.concatenate([qi, extra]))
    ki = np.unique(np.concatenate([ki, extra]))
    return qi.astype(np.int64), ki.astype(np.int64)
