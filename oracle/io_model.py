"""Closed-form HBM traffic and FLOP models (test infrastructure).

Element counts (not bytes) of HBM reads + writes for one head, reconstructed
from the prose of the CS324 Lecture 8 notes, section 5.1 (standard attention),
section 5.5 (the tiled algorithm's count; Theorem 2's displayed formula is lost
in the extraction) and exercise 4, whose printed totals the tests reproduce.

  standard forward   4N^2 + 4Nd     (S written, read; P written, read; Q, K, V
                                     read; O written -- section 5.1)
  standard backward  7N^2 + 8Nd     (section 5.1)
  tiled, per (j, i) block pair, forward:  read Q_i, O_i, l_i, m_i and write
      O_i, l_i, m_i -> 3 B_r d + 4 B_r;  plus K, V read once and O, l, m
      initialised once -> 3Nd + 2N
  tiled, per pair, backward: read Q_i, O_i, dO_i, dQ_i, l_i, m_i and write
      dQ_i -> 5 B_r d + 2 B_r;  plus K, V read, dK, dV written and dQ
      initialised once -> 5Nd
  so forward + backward = T_c (8Nd + 6N) + 8Nd + 2N with T_c = ceil(N / B_c).

The forward/backward split of the tiled count is a reading (only the totals
are printed).  FLOPs: one head's standard forward + backward matmuls are
12 N^2 d and the recomputing version 14 N^2 d (section 5.4); the credited
throughput metric counts 4 N^2 d for the forward (halved when causal) and
2.5x that for the backward.

``second_version_uncached`` is the traffic model of "FlashAttention and GPU
memory", section 14 (lab bench): each Q block read once, K and V read once per
Q block, O written once, no credit for L2.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import math

from .tiled import block_sizes

__all__ = [
    "standard_io",
    "flash_io",
    "flash_io_causal_forward",
    "second_version_uncached",
    "matmul_flops_standard",
    "matmul_flops_recompute",
    "credited_flops",
    "intensity_qkt",
]


def standard_io(n: int, d: int, backward: bool = True) -> int:
    """HBM elements moved by standard attention (forward [+ backward])."""
    fwd = 4 * n * n + 4 * n * d
    return fwd + (7 * n * n + 8 * n * d if backward else 0)


def flash_io(n: int, d: int, m_sram: int, backward: bool = True) -> int:
    """HBM elements moved by the tiled algorithm with K/V in the outer loop."""
    br, bc = block_sizes(m_sram, d)
    tc = math.ceil(n / bc)
    fwd = tc * (3 * n * d + 4 * n) + 3 * n * d + 2 * n
    if not backward:
        return fwd
    return fwd + tc * (5 * n * d + 2 * n) + 5 * n * d


def flash_io_causal_forward(n: int, d: int, br: int, bc: int) -> int:
    """Tiled forward count when blocks wholly in the future are skipped."""
    total = 3 * n * d + 2 * n
    for j0 in range(0, n, bc):
        for i0 in range(0, n, br):
            i1 = min(n, i0 + br)
            if j0 <= i1 - 1:
                total += 3 * (i1 - i0) * d + 4 * (i1 - i0)
    return total


def second_version_uncached(n: int, d: int, br: int, causal: bool = False) -> int:
    """Forward elements: Q once, K and V once per Q block, O written once.

    Causal: a Q block ending at row i1 reads only the K/V rows [0, i1).
    """
    total = 2 * n * d  # Q read, O written
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        kv_rows = i1 if causal else n
        total += 2 * kv_rows * d
    return total


def matmul_flops_standard(n: int, d: int) -> int:
    """Forward + backward matmul FLOPs of standard attention, one head."""
    return 12 * n * n * d


def matmul_flops_recompute(n: int, d: int) -> int:
    """Forward + backward matmul FLOPs when the backward recomputes S."""
    return 14 * n * n * d


def credited_flops(b: int, h: int, n: int, d: int, causal: bool):
    """(forward, backward) FLOPs credited by the throughput metric."""
    fwd = 4 * b * h * n * n * d
    if causal:
        fwd //= 2
    return fwd, fwd * 5 // 2


def intensity_qkt(n: int, d: int, bytes_per_el: int = 2):
    """(FLOPs, bytes, FLOP/byte) of one head's Q K^T with S written out.

    CS324 Lecture 8, exercise 1: read two N x d inputs, write the N x N
    output; 2 N^2 d FLOPs.
    """
    flops = 2 * n * d * n
    nbytes = bytes_per_el * (n * d + d * n + n * n)
    return flops, nbytes, flops / nbytes
