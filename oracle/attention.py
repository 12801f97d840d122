"""Standard attention and its chain-rule backward in fp64 (test infrastructure).

This is the plain definition that tiled/IO-aware attention reproduces exactly
up to rounding ("Lecture 8 . GPU Performance & FlashAttention", section 5.1
"why standard attention is slow" and section 5.7 "exact vs approximate";
"FlashAttention and GPU memory", sections 01 and 12).  S and P are
materialised in full for every head.

Conventions (readings where the pages leave a choice open):
  * tensors are [..., N, d]; any leading dims (batch, heads) are independent;
  * S = scale * Q K^T, the scale is an explicit argument;
  * causal: key j is visible to query i iff j <= i (the pages only say that
    blocks lying wholly in a query block's future are skipped, section 5.3);
  * LSE_i = m_i + ln(l_i), natural log, over the scaled and masked scores
    (the pages store m and l separately, section 5.4; LSE carries the same
    information in one number);
  * the backward formulas are lost in the page extraction around section
    5.4; what is used here is the textbook derivative of S -> softmax -> PV,
    consistent with the D identity stated there.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import torch

__all__ = [
    "scores",
    "softmax_rows",
    "attention_forward",
    "attention_forward_keys",
    "attention_backward",
    "attention_forward_backward",
    "visible_from_blocks",
    "attention_forward_backward_masked",
    "per_head",
]

_F64 = torch.float64


def _as64(x) -> torch.Tensor:
    t = torch.as_tensor(x)
    if t.dtype != _F64:
        t = t.to(_F64)
    return t


def scores(q, k, scale: float, causal: bool) -> torch.Tensor:
    """S = scale * Q K^T, with -inf above the diagonal when causal.

    Section 5.1 of the CS324 Lecture 8 notes (step 1 of standard attention);
    causal visibility j <= i as described in section 5.3 there.
    """
    q, k = _as64(q), _as64(k)
    s = scale * (q @ k.transpose(-1, -2))
    if causal:
        nq, nk = s.shape[-2], s.shape[-1]
        future = torch.ones(nq, nk, dtype=torch.bool).triu(diagonal=1)
        s = s.masked_fill(future, float("-inf"))
    return s


def softmax_rows(s: torch.Tensor):
    """Safe softmax over the last axis: returns (P, m, l).

    The row maximum is subtracted before exponentiation so that large scores
    do not overflow (CS324 Lecture 8, section 5.1).  m is the row max,
    l = sum_j exp(S_ij - m_i), P = exp(S - m) / l.
    """
    m = s.max(dim=-1).values
    e = torch.exp(s - m.unsqueeze(-1))
    l = e.sum(dim=-1)
    p = e / l.unsqueeze(-1)
    return p, m, l


def attention_forward(q, k, v, scale: float, causal: bool = False):
    """O = softmax(scale Q K^T [+ mask]) V and LSE = m + ln l, in fp64.

    Three steps of standard attention (CS324 Lecture 8, section 5.1;
    "FlashAttention and GPU memory", section 04): scores, row softmax,
    weighted sum of V rows.
    """
    v = _as64(v)
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = p @ v
    lse = m + torch.log(l)
    return o, lse


def attention_forward_keys(q, k, v, scale: float, causal: bool, lo: int, hi: int):
    """O and LSE of every row over the keys lo <= j < hi only, in fp64.

    One part of a row as the Flash-Decoding split produces it (CS324 Lecture
    8, section 8.2): the three steps of standard attention with the keys
    outside the part masked like future keys.  A row that sees no key of
    the part has nothing to normalise: O = 0 and LSE = -inf (the identity of
    the merge, exercise 3).
    """
    v = _as64(v)
    s = scores(q, k, scale, causal)
    kidx = torch.arange(s.shape[-1])
    s = s.masked_fill((kidx < lo) | (kidx >= hi), float("-inf"))
    m = s.max(dim=-1).values
    empty = m == float("-inf")
    e = torch.exp(s - torch.where(empty, torch.zeros_like(m), m).unsqueeze(-1))
    l = e.sum(dim=-1)
    p = e / torch.where(empty, torch.ones_like(l), l).unsqueeze(-1)
    o = p @ v
    lse = torch.where(empty, torch.full_like(m, float("-inf")), m + torch.log(l))
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool = False):
    """dQ, dK, dV of L = sum(dO * O) by the explicit chain rule, in fp64.

    With P stored (the standard backward the CS324 Lecture 8 notes contrast
    with recomputation in section 5.4):
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D 1^T)
        dQ = scale * dS K
        dK = scale * dS^T Q
    D is formed from P and dP by its definition here; the identity
    D_i = sum_k dO_ik O_ik stated in section 5.4 is checked separately.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    s = scores(q, k, scale, causal)
    p, _, _ = softmax_rows(s)
    dv = p.transpose(-1, -2) @ do
    dp = do @ v.transpose(-1, -2)
    dsum = (p * dp).sum(dim=-1, keepdim=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.transpose(-1, -2) @ q)
    return dq, dk, dv


def attention_forward_backward(q, k, v, do, scale: float, causal: bool = False):
    """Forward and backward sharing one materialised P (fp64).

    Returns (O, LSE, dQ, dK, dV).  Same formulas as ``attention_forward`` and
    ``attention_backward``; computing P once halves the oracle's cost.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    s = scores(q, k, scale, causal)
    p, m, l = softmax_rows(s)
    del s
    o = p @ v
    lse = m + torch.log(l)
    dv = p.transpose(-1, -2) @ do
    dp = do @ v.transpose(-1, -2)
    dsum = (p * dp).sum(dim=-1, keepdim=True)
    ds = p * (dp - dsum)
    del p, dp
    dq = scale * (ds @ k)
    dk = scale * (ds.transpose(-1, -2) @ q)
    return o, lse, dq, dk, dv


def visible_from_blocks(block_mask, n: int, block: int) -> torch.Tensor:
    """Element visibility [n, n] of a block mask [nb, nb] of block x block tiles.

    Block-sparse attention ("FlashAttention and GPU memory", section 10;
    CS324 Lecture 8, section 5.7): query i may see key j only if the tile
    (i // block, j // block) is set.
    """
    bm = torch.as_tensor(block_mask) != 0
    idx = torch.arange(n) // block
    return bm[idx.unsqueeze(1), idx.unsqueeze(0)]


def attention_forward_backward_masked(q, k, v, do, scale: float, causal: bool, visible):
    """Standard attention and its chain-rule backward with an extra mask (fp64).

    Scores with ``visible[i, j]`` False are -inf, like future keys, before
    the softmax; everything else is ``attention_forward_backward``.  A row
    that sees no key at all has nothing to normalise: its O is 0, its LSE
    -inf and it contributes nothing to any gradient (its dQ is 0).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    s = scores(q, k, scale, causal).masked_fill(~torch.as_tensor(visible), float("-inf"))
    m = s.max(dim=-1).values
    empty = m == float("-inf")
    e = torch.exp(s - torch.where(empty, torch.zeros_like(m), m).unsqueeze(-1))
    l = e.sum(dim=-1)
    p = e / torch.where(empty, torch.ones_like(l), l).unsqueeze(-1)
    o = p @ v
    lse = torch.where(empty, torch.full_like(m, float("-inf")), m + torch.log(l))
    dv = p.transpose(-1, -2) @ do
    dp = do @ v.transpose(-1, -2)
    dsum = (p * dp).sum(dim=-1, keepdim=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.transpose(-1, -2) @ q)
    return o, lse, dq, dk, dv


def per_head(fn, tensors, *args, heads_per_chunk: int = 16, **kw):
    """Apply ``fn`` to [B, H, N, d] inputs a few heads at a time.

    Heads are independent, so slicing the flattened B*H axis ("batch-sliced")
    bounds the memory of the materialised N x N matrices without changing any
    value.  Returns the outputs reassembled to their [B, H, ...] shapes.
    """
    ts = [_as64(t) for t in tensors]
    lead = ts[0].shape[:-2]
    flat = [t.reshape(-1, *t.shape[-2:]) for t in ts]
    nheads = flat[0].shape[0]
    outs = None
    for h0 in range(0, nheads, heads_per_chunk):
        part = fn(*[t[h0:h0 + heads_per_chunk] for t in flat], *args, **kw)
        if not isinstance(part, tuple):
            part = (part,)
        if outs is None:
            outs = [[] for _ in part]
        for acc, piece in zip(outs, part):
            acc.append(piece)
    res = tuple(torch.cat(acc, dim=0) for acc in outs)
    return tuple(r.reshape(*lead, *r.shape[1:]) for r in res)
