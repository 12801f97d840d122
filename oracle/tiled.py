"""Tiled attention models in fp64 (test infrastructure).

Two forward orders and the recomputing backward, written as plain loops over
blocks so that the algorithm can be compared against the whole-matrix
definition in ``oracle.attention``.  Reads and writes of the arrays that live
in "HBM" are counted in elements, which lets the tests compare the counts with
the closed-form IO model.

  * ``forward_outer_kv``: outer loop over K/V blocks, inner loop over Q
    blocks; O, l, m make a round trip through HBM for every (j, i) pair and O
    is kept normalised between steps (CS324 Lecture 8 notes, section 5.3,
    "Algorithm 1", and the block-size rule B_c = ceil(M/4d),
    B_r = min(ceil(M/4d), d) stated there).  Causal: a block lying wholly in
    the query block's future is neither read nor computed (same section, and
    section 5.7 on block-sparse attention).
  * ``forward_outer_q``: one Q block at a time, inner loop over K/V blocks,
    unnormalised accumulator divided once at the end ("Stanford CS336 Lecture
    5: GPUs", section 7 sketch; CS324 Lecture 8 section 8.1 on the second
    version dividing only at the end).
  * ``backward_recompute``: saves only O and the row statistics; each S and P
    block is recomputed from Q, K and the statistics and used at once (CS324
    Lecture 8, section 5.4; "FlashAttention and GPU memory", section 09).
    D_i is taken from the identity D_i = sum_k dO_ik O_ik of section 5.4.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "block_sizes",
    "IOCount",
    "forward_outer_kv",
    "forward_outer_q",
    "backward_recompute",
]

_F64 = torch.float64


def block_sizes(m_sram: int, d: int):
    """(B_r, B_c) from on-chip capacity M in elements (CS324 L8 section 5.3)."""
    bc = math.ceil(m_sram / (4 * d))
    return min(bc, d), bc


@dataclass
class IOCount:
    """Elements read from / written to HBM, and computed (i, j) block pairs."""
    reads: int = 0
    writes: int = 0
    pairs: int = 0

    @property
    def total(self) -> int:
        return self.reads + self.writes


def _visible(i0, i1, j0, causal):
    """True if some key of the block starting at j0 is visible to rows i0..i1-1."""
    return (not causal) or j0 <= i1 - 1


def _mask_block(s, i0, j0, causal):
    if not causal:
        return s
    qi = torch.arange(i0, i0 + s.shape[0]).unsqueeze(1)
    kj = torch.arange(j0, j0 + s.shape[1]).unsqueeze(0)
    return s.masked_fill(kj > qi, float("-inf"))


def forward_outer_kv(q, k, v, scale, causal, br, bc, io: IOCount | None = None, block_mask=None):
    """Tiled forward, K/V outer loop; returns (O, m, l) for one head [N, d].

    ``block_mask`` ([ceil(N/br), ceil(N/bc)], optional): block-sparse
    attention (section 5.7; "FlashAttention and GPU memory", section 10) --
    a block pair whose entry is 0 is neither read nor computed, exactly like
    a block in a query block's future.  A row that sees no key at all keeps
    l = 0, m = -inf and O = 0.
    """
    q, k, v = (t.to(_F64) for t in (q, k, v))
    n, d = q.shape
    io = io if io is not None else IOCount()
    o = torch.zeros(n, d, dtype=_F64)
    l = torch.zeros(n, dtype=_F64)
    m = torch.full((n,), float("-inf"), dtype=_F64)
    io.writes += n * d + 2 * n  # initialise O, l, m in HBM
    for j0 in range(0, n, bc):
        j1 = min(n, j0 + bc)
        kj, vj = k[j0:j1], v[j0:j1]
        io.reads += 2 * (j1 - j0) * d
        for i0 in range(0, n, br):
            i1 = min(n, i0 + br)
            if not _visible(i0, i1, j0, causal):
                continue
            if block_mask is not None and not block_mask[i0 // br][j0 // bc]:
                continue
            rows = i1 - i0
            io.reads += 2 * rows * d + 2 * rows  # Q_i, O_i, l_i, m_i
            io.pairs += 1
            s = _mask_block(scale * (q[i0:i1] @ kj.T), i0, j0, causal)
            mt = s.max(dim=1).values
            # a row with every key of this block masked has mt = -inf; it
            # contributes nothing (exp(-inf) = 0) and must not produce NaN.
            mt_safe = torch.where(torch.isinf(mt), torch.zeros_like(mt), mt)
            pt = torch.exp(s - mt_safe.unsqueeze(1))
            lt = pt.sum(dim=1)
            mi, li = m[i0:i1], l[i0:i1]
            m_new = torch.maximum(mi, mt)
            a = torch.where(torch.isinf(mi), torch.zeros_like(mi), torch.exp(mi - m_new))
            b = torch.where(torch.isinf(mt), torch.zeros_like(mt), torch.exp(mt_safe - m_new))
            l_new = a * li + b * lt
            den = torch.where(l_new > 0, l_new, torch.ones_like(l_new))
            o[i0:i1] = ((li * a).unsqueeze(1) * o[i0:i1] + b.unsqueeze(1) * (pt @ vj)) / den.unsqueeze(1)
            l[i0:i1] = l_new
            m[i0:i1] = m_new
            io.writes += rows * d + 2 * rows  # O_i, l_i, m_i
    return o, m, l


def forward_outer_q(q, k, v, scale, causal, br, bc, io: IOCount | None = None):
    """Tiled forward, Q outer loop, unnormalised accumulator; (O, LSE).

    ``io`` counts the elements of the N x d matrices that the loop moves:
    Q_i read once per Q block, K_j and V_j read once per visited (i, j)
    pair, O_i written once.  The row statistics (LSE, N elements written
    once) are left out of the count, as in the lab-bench traffic model of
    "FlashAttention and GPU memory", section 14.
    """
    q, k, v = (t.to(_F64) for t in (q, k, v))
    n, d = q.shape
    io = io if io is not None else IOCount()
    o = torch.empty(n, d, dtype=_F64)
    lse = torch.empty(n, dtype=_F64)
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        rows = i1 - i0
        qi = q[i0:i1]
        io.reads += rows * d
        m = torch.full((rows,), float("-inf"), dtype=_F64)
        l = torch.zeros(rows, dtype=_F64)
        acc = torch.zeros(rows, d, dtype=_F64)
        for j0 in range(0, n, bc):
            if not _visible(i0, i1, j0, causal):
                break
            j1 = min(n, j0 + bc)
            kj, vj = k[j0:j1], v[j0:j1]
            io.reads += 2 * (j1 - j0) * d
            io.pairs += 1
            s = _mask_block(scale * (qi @ kj.T), i0, j0, causal)
            m_new = torch.maximum(m, s.max(dim=1).values)
            # rows still without a visible key keep m = -inf; use base 0 there
            base = torch.where(torch.isinf(m_new), torch.zeros_like(m_new), m_new)
            p = torch.exp(s - base.unsqueeze(1))
            alpha = torch.where(torch.isinf(m), torch.zeros_like(m), torch.exp(m - base))
            l = alpha * l + p.sum(dim=1)
            acc = alpha.unsqueeze(1) * acc + p @ vj
            m = m_new
        o[i0:i1] = acc / l.unsqueeze(1)
        io.writes += rows * d
        lse[i0:i1] = m + torch.log(l)
    return o, lse


def backward_recompute(q, k, v, o, do, lse, scale, causal, br, bc,
                       io: IOCount | None = None):
    """Recomputing backward for one head; returns (dQ, dK, dV).

    K/V blocks in the outer loop, Q blocks inside; P_ij is rebuilt from
    scale*Q_i K_j^T and the saved LSE_i, and dQ_i makes a round trip through
    HBM per pair, as in the tiled forward above.
    """
    q, k, v, o, do, lse = (t.to(_F64) for t in (q, k, v, o, do, lse))
    n, d = q.shape
    io = io if io is not None else IOCount()
    dq = torch.zeros(n, d, dtype=_F64)
    dk = torch.zeros(n, d, dtype=_F64)
    dv = torch.zeros(n, d, dtype=_F64)
    io.writes += n * d  # initialise dQ
    for j0 in range(0, n, bc):
        j1 = min(n, j0 + bc)
        kj, vj = k[j0:j1], v[j0:j1]
        dkj = torch.zeros(j1 - j0, d, dtype=_F64)
        dvj = torch.zeros(j1 - j0, d, dtype=_F64)
        io.reads += 2 * (j1 - j0) * d
        for i0 in range(0, n, br):
            i1 = min(n, i0 + br)
            if not _visible(i0, i1, j0, causal):
                continue
            rows = i1 - i0
            # Q_i, O_i, dO_i, dQ_i and the two row statistics
            io.reads += 4 * rows * d + 2 * rows
            io.pairs += 1
            s = _mask_block(scale * (q[i0:i1] @ kj.T), i0, j0, causal)
            p = torch.exp(s - lse[i0:i1].unsqueeze(1))
            dvj += p.T @ do[i0:i1]
            dp = do[i0:i1] @ vj.T
            di = (do[i0:i1] * o[i0:i1]).sum(dim=1, keepdim=True)
            ds = p * (dp - di)
            dq[i0:i1] += scale * (ds @ kj)
            dkj += scale * (ds.T @ q[i0:i1])
            io.writes += rows * d  # dQ_i
        dk[j0:j1] = dkj
        dv[j0:j1] = dvj
        io.writes += 2 * (j1 - j0) * d
    return dq, dk, dv
