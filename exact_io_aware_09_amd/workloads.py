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


def make_trending_inputs(shape, dtype, seed: int, pattern: str, rise: float):
    """(Q, K, V, dO) whose scores change steeply along the keys.

    A seeded direction u (entries +-1) is shared by every query and key:
    Q[i] = a_i u + n/4 and K[j] = r_j u + n/4 with n ~ N(0, 1), so that the
    score of (i, j) is about a_i r_j d / sqrt(d) plus noise.  ``rise`` is the
    total change of r_j u.u / sqrt(d) over the sequence.

    * ``"ramp"``: r_j rises linearly over the keys (centred on 0), a_i = 1;
      every row's largest scores sit at its last visible keys.
    * ``"spike"``: r_j = 0 except two late keys (N/2 + 3 and N - 5) at
      r = rise / 2 and rise; a_i = 1.
    * ``"mixed"``: the ramp, with a_i = (i mod 3) - 1, so rows alternate
      between rising, flat and falling scores.

    V and dO are N(0, 1).  Values are rounded to ``dtype`` like
    ``make_inputs``.
    """
    B, H, N, d = shape
    g = torch.Generator("cpu").manual_seed(int(seed))
    u = torch.randint(0, 2, (d,), generator=g).to(torch.float32) * 2 - 1
    nq = torch.randn(tuple(shape), generator=g) / 4
    nk = torch.randn(tuple(shape), generator=g) / 4
    v = torch.randn(tuple(shape), generator=g)
    do = torch.randn(tuple(shape), generator=g)
    step = rise / d ** 0.5
    j = torch.arange(N, dtype=torch.float32)
    if pattern == "spike":
        r = torch.zeros(N)
        for pos, frac in ((N // 2 + 3, 0.5), (N - 5, 1.0)):
            if 0 <= pos < N:
                r[pos] = step * frac
        a = torch.ones(N)
    elif pattern in ("ramp", "mixed"):
        r = step * (j / max(N - 1, 1) - 0.5)
        a = torch.ones(N) if pattern == "ramp" else (torch.arange(N) % 3 - 1).to(torch.float32)
    else:
        raise ValueError(f"unknown pattern {pattern!r}")
    q = a[:, None] * u[None, :] + nq
    k = r[:, None] * u[None, :] + nk
    return tuple(t.to(dtype) for t in (q, k, v, do))


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
