"""Attention with dropout on the softmax weights, fp64 (test infrastructure).

The fused kernel of the pages applies dropout to the attention weights after
the softmax and before the product with V ("FlashAttention and GPU memory",
section 07, which lists matmul, softmax, mask, dropout, matmul as one
program); the forward keeps only the state of the random number generator and
the backward regenerates the same mask from it instead of storing it ("FlashAttention
and GPU memory", section 09; "Lecture 8 . GPU Performance & FlashAttention",
CS324 notes, section 5.4).

Readings (the pages fix neither the generator, the layout of its draws, nor
the resolution of the keep test):

* Draws: one Philox4x32-10 block per 4 x 4 tile of (query, key) pairs of a
  head.  For query i and key j of head bh = b*H + h the counter is
  (j // 4, i // 4, bh, 0) and the key (seed mod 2^32, seed div 2^32); the
  element's draw u_ij in 0..255 is byte (j mod 4) (little-endian) of word
  (i mod 4) of the block.
* Keep test: element kept iff u_ij < t, where t = round((1 - p) * 256) for
  the probability p as a float32 (1 <= t <= 256).  p_eff = 1 - t/256 is the
  probability actually applied, and kept weights are scaled by 256/t, so the
  expected dropped weight equals the weight exactly.
* Forward: O = (P o Z) V * 256/t, Z the keep mask; LSE is the log-sum-exp of
  the scaled, masked scores, untouched by dropout (it normalises P).
* Backward: the textbook chain rule with Z fixed.  With Pd = P o Z * 256/t:
  dV = Pd^T dO;  dP = (dO V^T) o Z * 256/t;  D_i = sum_j P_ij dP_ij, which
  equals sum_k dO_ik O_ik (checked in tests);  dS = P o (dP - D);
  dQ = scale dS K;  dK = scale dS^T Q.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import _as64, scores, softmax_rows
from .philox import philox4x32_10

__all__ = ["keep_threshold", "draws", "keep_masks", "attention_forward_backward_dropout"]


def keep_threshold(p) -> int:
    """t = round((1 - p) * 256) for the float32 value of p; needs 1 <= t <= 256."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    t = int(np.floor((1.0 - p32) * 256.0 + 0.5))
    if t < 1:
        raise ValueError("dropout probability too close to 1: no element would be kept")
    return t


def draws(seed: int, bh: int, rows, cols) -> np.ndarray:
    """8-bit draws u_ij (uint8 [len(rows), len(cols)]) of head bh.

    One generator block per 4 x 4 tile of (query, key) pairs; see the module
    docstring for the counter and the byte of the block that (i, j) takes.
    """
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    cols = np.asarray(cols, dtype=np.uint64).reshape(1, -1)
    ctr = np.stack(np.broadcast_arrays(cols >> np.uint64(2), rows >> np.uint64(2),
                                       np.full_like(rows, bh), np.zeros_like(rows)), axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    blocks = philox4x32_10(ctr, key)                            # [rows, cols, 4] words
    wsel = np.broadcast_to((rows & np.uint64(3)).astype(np.intp)[..., None], blocks.shape[:2] + (1,))
    word = np.take_along_axis(blocks, wsel, axis=-1)[..., 0]
    shift = (np.uint64(8) * (cols & np.uint64(3))).astype(np.uint32)
    return ((word >> shift) & np.uint32(0xFF)).astype(np.uint8)


def keep_masks(seed: int, B: int, H: int, N: int, t: int) -> torch.Tensor:
    """Keep masks Z (bool [B, H, N, N]) of every head: u_ij < t."""
    idx = np.arange(N)
    z = np.empty((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            z[b, h] = draws(seed, b * H + h, idx, idx) < t
    return torch.from_numpy(z)


def attention_forward_backward_dropout(q, k, v, do, scale: float, causal: bool, keep, t: int):
    """O, LSE, dQ, dK, dV of attention with the weights dropped by ``keep``.

    ``keep`` is the bool keep mask (broadcastable to [..., N, N]) and t the
    keep threshold it was drawn with (kept weights scaled by 256/t).  Formulas
    as in the module docstring; S and P are materialised per call.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    z = torch.as_tensor(keep).to(torch.float64) * (256.0 / t)
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    del s
    pd = p * z
    o = pd @ v
    lse = m + torch.log(l)
    dv = pd.transpose(-1, -2) @ do
    dp = (do @ v.transpose(-1, -2)) * z
    dsum = (p * dp).sum(dim=-1, keepdim=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.transpose(-1, -2) @ q)
    return o, lse, dq, dk, dv
