"""Autograd wrapper: attention as a differentiable PyTorch op backed by the C ABI.

``flash_attention(q, k, v, causal=False, scale=None, dropout_p=0.0, seed=None)``
takes contiguous [B, H, N, d] tensors on the GPU (bfloat16 or float32) and
returns O; its backward runs the library's recomputing backward.  The pages
present the fused kernel as a replacement with the interface of the attention
call it replaces ("Lecture 8 . GPU Performance & FlashAttention", section 6.3),
which is what this provides: the forward keeps only O and the log-sum-exp for
the backward (section 5.4), plus the dropout seed when dropout is on.  Every
step runs in the HIP kernels; this module only passes tensors through.
"""
from __future__ import annotations

import torch

from . import attention as _att


class FlashAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float, dropout_p: float, seed: int):
        if dropout_p > 0.0:
            o, lse = _att.forward_dropout(q, k, v, scale, causal, dropout_p, seed)
        else:
            o, lse = _att.forward(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.dropout_p, ctx.seed = causal, scale, dropout_p, seed
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do.contiguous()
        if ctx.dropout_p > 0.0:
            dq, dk, dv = _att.backward_dropout(q, k, v, o, do, lse, ctx.scale, ctx.causal,
                                               ctx.dropout_p, ctx.seed)
        else:
            dq, dk, dv = _att.backward(q, k, v, o, do, lse, ctx.scale, ctx.causal)
        return dq, dk, dv, None, None, None, None


def flash_attention(q, k, v, causal: bool = False, scale: float | None = None,
                    dropout_p: float = 0.0, seed: int | None = None):
    """O = softmax(scale Q K^T [causal mask]) [dropout] V, differentiable in q, k, v.

    scale defaults to 1/sqrt(d).  With dropout, ``seed`` (64-bit) keys the
    generator; if None, one is drawn from torch's default CPU generator, so
    torch.manual_seed makes runs repeatable.
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    if dropout_p > 0.0 and seed is None:
        seed = int(torch.randint(0, 2**62, (1,)).item())
    return FlashAttentionFunction.apply(q, k, v, bool(causal), float(scale), float(dropout_p),
                                        int(seed or 0))
