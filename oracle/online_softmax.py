"""Online softmax statistics in fp64 (test infrastructure).

The running pair (m, l): m is the largest score seen so far and l is the sum
of exp(x - m) over the scores seen so far.  When a new maximum arrives the old
sum is moved to the new base by the factor exp(m_old - m_new) before the new
terms are added, so a row can be consumed in pieces and still yield the exact
normaliser.

Sources:
  * element-wise stream: "Stanford CS336 Lecture 5: GPUs", section 7
    (online softmax sketch);
  * block-wise update m_new = max(m, m~), l_new = e^(m-m_new) l + e^(m~-m_new) l~:
    CS324 Lecture 8 notes, section 5.2 (its displayed formula is lost in the
    extraction; the same update is restated in "FlashAttention and GPU
    memory", section 08);
  * merging two independently processed parts, with the output rescaled the
    same way: CS324 Lecture 8, exercises 3 and 7, and section 8.2
    (Flash-Decoding).

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

__all__ = [
    "stream",
    "blocks",
    "merge",
    "merge_with_output",
    "merge_parts",
    "softmax_from_stats",
]


def stream(xs: Iterable[float]) -> Tuple[float, float]:
    """Consume scores one at a time; return the final (m, l)."""
    m, l = -math.inf, 0.0
    for x in xs:
        m_new = max(m, x)
        # exp(-inf - finite) is 0: the empty prefix contributes nothing.
        l = l * (math.exp(m - m_new) if m != -math.inf else 0.0) + math.exp(x - m_new)
        m = m_new
    return m, l


def _block_stats(block: Sequence[float]) -> Tuple[float, float]:
    mb = max(block)
    return mb, sum(math.exp(x - mb) for x in block)


def merge(m1: float, l1: float, m2: float, l2: float) -> Tuple[float, float]:
    """Combine two partial (m, l) states into the state of their union.

    Symmetric in its two arguments (CS324 Lecture 8, exercise 3).  A part that
    has seen nothing is (-inf, 0) and leaves the other unchanged.
    """
    m = max(m1, m2)
    if m == -math.inf:
        return m, 0.0
    a = math.exp(m1 - m) if m1 != -math.inf else 0.0
    b = math.exp(m2 - m) if m2 != -math.inf else 0.0
    return m, l1 * a + l2 * b


def blocks(xs: Sequence[float], block: int) -> List[Tuple[float, float]]:
    """Read ``xs`` ``block`` scores at a time; return (m, l) after each block.

    Each block's own (m~, l~) is formed and folded into the running state with
    the block update of CS324 Lecture 8 section 5.2.
    """
    out = []
    m, l = -math.inf, 0.0
    for s in range(0, len(xs), block):
        mb, lb = _block_stats(xs[s:s + block])
        m, l = merge(m, l, mb, lb)
        out.append((m, l))
    return out


def merge_with_output(m1, l1, o1, m2, l2, o2):
    """Merge two partial (m, l, o) states where o is the *normalised* output.

    Each part's o_k = (sum_j exp(x_j - m_k) v_j) / l_k.  Un-normalise with
    l_k, move to the common base with exp(m_k - m), add, and normalise by the
    merged l (CS324 Lecture 8, exercise 7; section 8.2 on Flash-Decoding).
    ``o1`` and ``o2`` are sequences of floats (one output row).
    """
    m, l = merge(m1, l1, m2, l2)
    a = l1 * math.exp(m1 - m) if m1 != -math.inf else 0.0
    b = l2 * math.exp(m2 - m) if m2 != -math.inf else 0.0
    return m, l, [(a * x + b * y) / l for x, y in zip(o1, o2)]


def softmax_from_stats(xs: Sequence[float], m: float, l: float) -> List[float]:
    """softmax(x)_j = exp(x_j - m) / l once the whole row has been read."""
    return [math.exp(x - m) / l for x in xs]


def merge_parts(lse_parts, o_parts):
    """Merge S partial results of the same rows, part by part (fp64 torch).

    lse_parts: [S, ...] natural-log log-sum-exps of each part (-inf for a
    part with no key); o_parts: [S, ..., d] each part's output normalised
    over its own keys.  A part's running state is (m, l) = (L_s, 1), since
    e^{L_s} = l_s e^{m_s}; the parts are folded one after another with the
    update of ``merge`` (exercise 3) and the output is un-normalised, moved
    to the common base and re-normalised as in ``merge_with_output``
    (exercise 7, section 8.2).  Returns (LSE, O); a row whose parts are all
    empty gets LSE = -inf and O = 0.
    """
    import torch

    ninf = float("-inf")
    m = lse_parts[0].clone()
    l = torch.where(m == ninf, torch.zeros_like(m), torch.ones_like(m))
    o = o_parts[0].clone()
    for s in range(1, lse_parts.shape[0]):
        ms = lse_parts[s]
        mn = torch.maximum(m, ms)
        safe = torch.where(mn == ninf, torch.zeros_like(mn), mn)
        a = torch.where(m == ninf, torch.zeros_like(m), l * torch.exp(m - safe))
        b = torch.where(ms == ninf, torch.zeros_like(ms), torch.exp(ms - safe))
        ln = a + b
        den = torch.where(ln > 0, ln, torch.ones_like(ln))
        o = (a.unsqueeze(-1) * o + b.unsqueeze(-1) * o_parts[s]) / den.unsqueeze(-1)
        m, l = mn, ln
    lse = torch.where(l > 0, m + torch.log(torch.where(l > 0, l, torch.ones_like(l))), torch.full_like(m, ninf))
    return lse, o
