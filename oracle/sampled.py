"""The attention definition restricted to chosen rows (fp64, test infrastructure).

At long sequence lengths (N = 65,536) a full N x N score matrix per head is
out of reach for a CPU check, so these functions evaluate exactly the same
definitions as ``oracle.attention`` for selected query rows and selected key
rows only.  Rows of S and P are independent of each other, so each query row
is computed in full (all N keys) and nothing is approximated; the pages'
standard attention (CS324 Lecture 8, section 5.1) is simply evaluated a few
rows (or a chunk of rows) at a time.

For a key row j the gradients dK_j and dV_j sum over *every* query row i, and
each term needs that row's P_i (hence its full softmax statistics) and
D_i = sum_j P_ij dP_ij.  ``key_rows`` therefore streams all query rows in
chunks, materialising S, P and dP for one chunk at a time (memory
O(chunk * N)).  Causal: a query chunk only reaches keys up to its last row.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import torch

from .attention import softmax_rows

__all__ = ["query_rows", "key_rows"]

_F64 = torch.float64


def _masked_scores(q_rows, row_idx, k, scale, causal):
    """scale * q_rows K^T with -inf where key index > query index (causal)."""
    s = scale * (q_rows @ k.transpose(0, 1))
    if causal:
        kidx = torch.arange(k.shape[0])
        s = s.masked_fill(kidx.unsqueeze(0) > row_idx.unsqueeze(1), float("-inf"))
    return s


def query_rows(q, k, v, do, rows, scale: float, causal: bool):
    """O_i, LSE_i and dQ_i for the query rows ``rows`` of one head.

    q, k, v, do: [N, d] (any float dtype; upcast to fp64).  Each selected row
    gets its full score row, safe softmax, O_i = P_i V, LSE_i = m_i + ln l_i,
    and dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j with dP_i = dO_i V^T and
    D_i = sum_j P_ij dP_ij (chain rule, CS324 Lecture 8, section 5.4).
    """
    q, k, v, do = (t.to(_F64) for t in (q, k, v, do))
    rows = torch.as_tensor(rows, dtype=torch.long)
    s = _masked_scores(q[rows], rows, k, scale, causal)
    p, m, l = softmax_rows(s)
    o = p @ v
    lse = m + torch.log(l)
    dp = do[rows] @ v.transpose(0, 1)
    dsum = (p * dp).sum(dim=-1, keepdim=True)
    dq = scale * ((p * (dp - dsum)) @ k)
    return o, lse, dq


def key_rows(q, k, v, do, cols, scale: float, causal: bool, chunk: int = 512):
    """dK_j and dV_j for the key rows ``cols`` of one head, exactly.

    dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij Q_i over all query
    rows i (causal: i >= j), with dS = P * (dP - D).  Query rows are streamed
    in chunks of ``chunk``; for each chunk the full score rows are formed so
    that P and D are those of the complete softmax.
    """
    q, k, v, do = (t.to(_F64) for t in (q, k, v, do))
    cols = torch.as_tensor(cols, dtype=torch.long)
    n, d = q.shape
    dk = torch.zeros(cols.numel(), d, dtype=_F64)
    dv = torch.zeros(cols.numel(), d, dtype=_F64)
    cmin = int(cols.min()) if cols.numel() else n
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        if causal and r1 - 1 < cmin:
            continue  # every selected key is in these rows' future
        ridx = torch.arange(r0, r1)
        kend = r1 if causal else n  # causal rows never see keys past r1-1
        s = _masked_scores(q[r0:r1], ridx, k[:kend], scale, causal)
        p, _, _ = softmax_rows(s)
        dp = do[r0:r1] @ v[:kend].transpose(0, 1)
        dsum = (p * dp).sum(dim=-1, keepdim=True)
        ds = p * (dp - dsum)
        sel = cols < kend
        if not bool(sel.any()):
            continue
        csel = cols[sel]
        dv[sel] += p[:, csel].transpose(0, 1) @ do[r0:r1]
        dk[sel] += scale * (ds[:, csel].transpose(0, 1) @ q[r0:r1])
    return dk, dv
