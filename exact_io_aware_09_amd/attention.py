"""Tensor-level wrappers over the C ABI (torch supplies device memory and the stream).

``forward`` and ``backward`` check shapes/dtypes on the host, allocate the
outputs with ``torch.empty`` on the inputs' device and call ``fa_forward`` /
``fa_backward`` on the current HIP stream.  No arithmetic happens here.
"""
from __future__ import annotations

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.FA_BF16, torch.float32: _lib.FA_F32}


def _check(name, t, ref=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if ref is not None:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{name} must match Q in shape, dtype and device")


def _dims(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    return (*q.shape, _DTYPES[q.dtype])


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def forward(q, k, v, scale: float, causal: bool = False, out=None, lse=None):
    """Returns (O, LSE) for [B, H, N, d] inputs; LSE is float32 [B, H, N]."""
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d, dt = _dims(q)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", o, q)
    rc = _lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         lse_t.data_ptr(), B, H, N, d, scale, int(bool(causal)), dt,
                         _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward")
    return o, lse_t


def workspace_bytes(B, H, N, d, dtype) -> int:
    return _lib.fa_backward_workspace_bytes(B, H, N, d, _DTYPES[dtype])


def backward(q, k, v, o, do, lse, scale: float, causal: bool = False, workspace=None,
             dq=None, dk=None, dv=None):
    """Returns (dQ, dK, dV).  ``workspace``: optional uint8 device tensor."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, None if name == "q" else q)
    B, H, N, d, dt = _dims(q)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    need = _lib.fa_backward_workspace_bytes(B, H, N, d, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    rc = _lib.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                          B, H, N, d, scale, int(bool(causal)), dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_backward")
    return dq, dk, dv
