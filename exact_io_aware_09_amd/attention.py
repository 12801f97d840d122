"""Tensor-level wrappers over the C ABI (torch supplies device memory and the stream).

``forward`` and ``backward`` check shapes/dtypes on the host, allocate the
outputs with ``torch.empty`` on the inputs' device and call ``fa_forward`` /
``fa_backward`` on the current HIP stream.  No arithmetic happens here.
"""
from __future__ import annotations

import ctypes

import numpy as np
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


def _check_lse(lse, q):
    B, H, N = q.shape[:3]
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on the inputs' device")


def _check_workspace(ws, need, q):
    if (not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous()
            or ws.device != q.device or ws.numel() < need):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {need} bytes "
                         "on the inputs' device")


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
    _check_lse(lse_t, q)
    rc = _lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         lse_t.data_ptr(), B, H, N, d, scale, int(bool(causal)), dt,
                         _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward")
    return o, lse_t


def forward_split(q, k, v, scale: float, causal: bool = False, splits: int = 2, workspace=None,
                  out=None, lse=None):
    """``forward`` through the split-KV entry point (bfloat16 for splits > 1)."""
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d, dt = _dims(q)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", o, q)
    _check_lse(lse_t, q)
    need = _lib.fa_forward_split_workspace_bytes(B, H, N, d, splits, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
    _check_workspace(ws, need, q)
    rc = _lib.fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse_t.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                               B, H, N, d, scale, int(bool(causal)), splits, dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward_split")
    return o, lse_t


def merge_partials(o_parts, lse_parts, dtype=torch.bfloat16):
    """Merge float32 partial results [S, B, H, N, d] / [S, B, H, N] into (O, LSE)."""
    if o_parts.dim() != 5 or o_parts.dtype != torch.float32 or not o_parts.is_contiguous():
        raise ValueError("o_parts must be contiguous float32 [S, B, H, N, d]")
    S, B, H, N, d = o_parts.shape
    if lse_parts.shape != (S, B, H, N) or lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be contiguous float32 [S, B, H, N]")
    o = torch.empty((B, H, N, d), dtype=dtype, device=o_parts.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    rc = _lib.fa_merge_partials(o_parts.data_ptr(), lse_parts.data_ptr(), S, o.data_ptr(),
                                lse.data_ptr(), B, H, N, d, _DTYPES[dtype], _stream(o_parts.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_merge_partials")
    return o, lse


def _mask_check(block_mask, q):
    N = q.shape[2]
    nb = (N + 127) // 128
    if (block_mask.shape != (nb, nb) or block_mask.dtype != torch.int32 or not block_mask.is_contiguous()
            or block_mask.device != q.device):
        raise ValueError(f"block_mask must be contiguous int32 [{nb}, {nb}] on the inputs' device")


def forward_sparse(q, k, v, block_mask, scale: float, causal: bool = False):
    """Block-sparse forward: (O, LSE); ``block_mask`` int32 [ceil(N/128)]^2 on the device."""
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d, dt = _dims(q)
    _mask_check(block_mask, q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.fa_forward_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), block_mask.data_ptr(), B, H, N, d, scale,
                                int(bool(causal)), dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward_sparse")
    return o, lse


def backward_sparse(q, k, v, o, do, lse, block_mask, scale: float, causal: bool = False):
    """Block-sparse backward: (dQ, dK, dV)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, None if name == "q" else q)
    B, H, N, d, dt = _dims(q)
    _mask_check(block_mask, q)
    _check_lse(lse, q)
    ws = torch.empty(_lib.fa_backward_workspace_bytes(B, H, N, d, dt), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    rc = _lib.fa_backward_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 do.data_ptr(), lse.data_ptr(), block_mask.data_ptr(),
                                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                 ws.numel(), B, H, N, d, scale, int(bool(causal)), dt,
                                 _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_backward_sparse")
    return dq, dk, dv


class SparseSchedule:
    """A balanced block-sparse schedule: the int32 array ``fa_sparse_schedule``
    wrote (``host``) and, once ``to(device)`` has run, its device copy."""

    def __init__(self, host: np.ndarray):
        self.host = host
        self.device_copy = None

    def field(self, name: str) -> int:
        return int(self.host[_lib.FA_SCHED_FIELDS[name]])

    def to(self, device):
        self.device_copy = torch.from_numpy(self.host).to(device)
        return self

    def _section(self, off, count, width=4):
        o = self.field(off)
        return self.host[o:o + width * count].reshape(count, width) if width > 1 else \
            self.host[o:o + count]

    def rows(self):
        """Row items [n, 4]: tile, list offset, tile count, slot word."""
        return self._section("OFF_ROWS", self.field("N_ROWS"))

    def cols(self):
        return self._section("OFF_COLS", self.field("N_COLS"))

    def long_rows(self):
        return self._section("OFF_LONG_ROWS", self.field("N_LONG_ROWS"))

    def long_cols(self):
        return self._section("OFF_LONG_COLS", self.field("N_LONG_COLS"))

    def lists(self):
        return self._section("OFF_LISTS", self.field("LIST_LEN"), width=1)


def sparse_schedule(block_mask, N: int, causal: bool, B: int, H: int, seg_tiles: int = 0):
    """Builds the balanced schedule of a tile mask (host int32 [nb, nb], numpy or CPU tensor)."""
    if isinstance(block_mask, torch.Tensor):
        block_mask = block_mask.detach().cpu().numpy()
    m = np.ascontiguousarray(block_mask, dtype=np.int32)
    nb = (N + 127) // 128
    if m.shape != (nb, nb):
        raise ValueError(f"block_mask must be [{nb}, {nb}]")
    needed = ctypes.c_size_t(0)
    rc = _lib.fa_sparse_schedule(m.ctypes.data, N, int(bool(causal)), B, H, seg_tiles, None, 0,
                                 ctypes.addressof(needed))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_sparse_schedule")
    host = np.zeros(needed.value, dtype=np.int32)
    rc = _lib.fa_sparse_schedule(m.ctypes.data, N, int(bool(causal)), B, H, seg_tiles,
                                 host.ctypes.data, host.size, ctypes.addressof(needed))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_sparse_schedule")
    return SparseSchedule(host)


def _sched_check(sched, q):
    if not isinstance(sched, SparseSchedule) or sched.device_copy is None \
            or sched.device_copy.device != q.device:
        raise ValueError("schedule must be a SparseSchedule copied to the inputs' device")


def forward_sparse_balanced(q, k, v, sched, scale: float, causal: bool = False):
    """Block-sparse forward over a balanced schedule: (O, LSE)."""
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d, dt = _dims(q)
    _sched_check(sched, q)
    need = _lib.fa_sparse_workspace_bytes(sched.host.ctypes.data, B, H, N, d, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.fa_forward_sparse_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), sched.host.ctypes.data,
                                         sched.device_copy.data_ptr(), ws.data_ptr(), ws.numel(),
                                         B, H, N, d, scale, int(bool(causal)), dt,
                                         _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward_sparse_balanced")
    return o, lse


def backward_sparse_balanced(q, k, v, o, do, lse, sched, scale: float, causal: bool = False):
    """Block-sparse backward over a balanced schedule: (dQ, dK, dV)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, None if name == "q" else q)
    B, H, N, d, dt = _dims(q)
    _sched_check(sched, q)
    _check_lse(lse, q)
    need = _lib.fa_sparse_workspace_bytes(sched.host.ctypes.data, B, H, N, d, 1)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    rc = _lib.fa_backward_sparse_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          do.data_ptr(), lse.data_ptr(), sched.host.ctypes.data,
                                          sched.device_copy.data_ptr(), dq.data_ptr(),
                                          dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                                          B, H, N, d, scale, int(bool(causal)), dt,
                                          _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_backward_sparse_balanced")
    return dq, dk, dv


def forward_dropout(q, k, v, scale: float, causal: bool, p_drop: float, seed: int):
    """Forward with dropout on the weights: (O, LSE); bfloat16 [B, H, N, d] inputs."""
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d, dt = _dims(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.fa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), B, H, N, d, scale, int(bool(causal)), p_drop,
                                 seed, dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward_dropout")
    return o, lse


def backward_dropout(q, k, v, o, do, lse, scale: float, causal: bool, p_drop: float, seed: int):
    """Backward of ``forward_dropout`` with the same p_drop and seed: (dQ, dK, dV)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, None if name == "q" else q)
    B, H, N, d, dt = _dims(q)
    _check_lse(lse, q)
    ws = torch.empty(_lib.fa_backward_workspace_bytes(B, H, N, d, dt), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    rc = _lib.fa_backward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), ws.data_ptr(), ws.numel(), B, H, N, d, scale,
                                  int(bool(causal)), p_drop, seed, dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_backward_dropout")
    return dq, dk, dv


def quantize_fp8(x, keys: bool = False):
    """E4M3 codes and block exponent bytes (uint8 device tensors) of a bfloat16 [B, H, N, d] tensor.

    keys=False (Q, K): codes [B, H, N, d], exponents [B, H, Np, d/32] (rows >= N: padding).
    keys=True (V): codes [B, H, d, Np] (transposed, keys padded to Np = 64 * ceil(N/64)),
    exponents [B, H, Np/32, d].
    """
    _check("x", x)
    B, H, N, d, dt = _dims(x)
    if dt != _lib.FA_BF16:
        raise ValueError("fa_quantize_fp8 takes bfloat16 input")
    layout = _lib.FA_FP8_KEYS if keys else _lib.FA_FP8_ROWS
    Np = -(-N // 64) * 64
    shape8 = (B, H, d, Np) if keys else (B, H, N, d)
    shapes = (B, H, Np // 32, d) if keys else (B, H, Np, d // 32)
    x8 = torch.empty(shape8, dtype=torch.uint8, device=x.device)
    xs = torch.empty(shapes, dtype=torch.uint8, device=x.device)
    assert x8.numel() == _lib.fa_fp8_bytes(B, H, N, d, layout)
    assert xs.numel() == _lib.fa_fp8_scale_bytes(B, H, N, d, layout)
    rc = _lib.fa_quantize_fp8(x.data_ptr(), x8.data_ptr(), xs.data_ptr(), B, H, N, d, layout,
                              _stream(x.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_quantize_fp8")
    return x8, xs


def forward_fp8(q8, qs, k8, ks, v8, vs, scale: float, causal: bool = False):
    """FP8 forward from ``quantize_fp8`` outputs: (O bfloat16, LSE float32)."""
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("qs", qs), ("k8", k8), ("ks", ks), ("v8", v8), ("vs", vs)):
        _check(name, t)
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must be uint8")
    Np = -(-N // 64) * 64
    if k8.shape != q8.shape or qs.shape != (B, H, Np, d // 32) or ks.shape != qs.shape:
        raise ValueError("q8/k8 must be [B, H, N, d] with scales [B, H, Np, d/32]")
    if v8.shape != (B, H, d, Np) or vs.shape != (B, H, Np // 32, d):
        raise ValueError("v8 must be [B, H, d, Np] with scales [B, H, Np/32, d]")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    rc = _lib.fa_forward_fp8(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                             v8.data_ptr(), vs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                             scale, int(bool(causal)), _stream(q8.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_forward_fp8")
    return o, lse


def workspace_bytes(B, H, N, d, dtype) -> int:
    return _lib.fa_backward_workspace_bytes(B, H, N, d, _DTYPES[dtype])


def backward(q, k, v, o, do, lse, scale: float, causal: bool = False, workspace=None,
             dq=None, dk=None, dv=None):
    """Returns (dQ, dK, dV).  ``workspace``: optional uint8 device tensor."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, None if name == "q" else q)
    B, H, N, d, dt = _dims(q)
    _check_lse(lse, q)
    need = _lib.fa_backward_workspace_bytes(B, H, N, d, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    _check_workspace(ws, need, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q)
    rc = _lib.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                          B, H, N, d, scale, int(bool(causal)), dt, _stream(q.device))
    if rc != _lib.FA_OK:
        raise _lib.FAError(rc, "fa_backward")
    return dq, dk, dv
