"""FP8 block quantisation and attention of quantised inputs, fp64 (test infrastructure).

The third version of the kernel runs attention in 8-bit floating point with
block quantisation ("Lecture 8 . GPU Performance & FlashAttention", CS324
notes, section 8.1; "FlashAttention and GPU memory", section 11).  The pages
name the technique only; the readings below fix it.

Readings:

* Element format: OCP 8-bit floating point E4M3 ("E4M3FN": 1 sign, 4
  exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
  largest finite value 448), round to nearest, ties to even.
* Blocks: 32 consecutive elements along the axis a product contracts over,
  sharing one power-of-two scale 2^e stored as an 8-bit biased exponent
  (e + 127): for Q and K, 32 consecutive head dimensions of a row; for V,
  32 consecutive keys of one head dimension.  e is the smallest integer with
  amax <= 448 * 2^e (amax = largest magnitude in the block; e = 0 for an
  all-zero block), clamped to [-127, 127]; an element x is stored as
  E4M3(x / 2^e), which never overflows.
* The attention of quantised inputs is the plain definition applied to the
  dequantised values Q^, K^, V^: O = softmax(scale Q^ K^T) V^, LSE its
  log-sum-exp.  A kernel that also rounds the softmax weights to E4M3 before
  the product with V (as the fused FP8 kernel does) differs from it by at
  most the relative rounding of those weights.

Only ``tests/``, ``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .attention import attention_forward

__all__ = ["E4M3_MAX", "e4m3_round", "e4m3_encode", "e4m3_decode", "block_exponent",
           "quantize_blocks", "quantize_rows", "quantize_keys", "attention_forward_fp8"]

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6   # smallest normal: 2^-6
_MANT_BITS = 3


def e4m3_round(x) -> np.ndarray:
    """Round fp64 values to the nearest E4M3 value (ties to even); |x| <= 464 required.

    Normal numbers 2^E * 1.mmm (E >= -6) have spacing 2^(E-3); below 2^-6 the
    subnormals have the fixed spacing 2^-9.  Rounding to a multiple of the
    spacing with numpy's round-half-even gives the E4M3 value; a result of
    2^(E+1) simply moves to the next binade.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 464.0) or np.any(~np.isfinite(x)):
        raise ValueError("value outside the E4M3 range")
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, _MIN_NORMAL_EXP)
    spacing = np.exp2(e - _MANT_BITS)
    r = np.round(ax / spacing) * spacing
    return np.where(ax > 0, np.copysign(r, x), 0.0 * x)


def e4m3_encode(v) -> np.ndarray:
    """Bit patterns (uint8) of E4M3 values (as returned by e4m3_round)."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint8)
    sub = a < 2.0 ** _MIN_NORMAL_EXP
    # subnormal: a = m * 2^-9, m in 0..7, exponent field 0
    m_sub = np.round(a / 2.0 ** -9).astype(np.int64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    m_norm = np.round((a / np.exp2(e) - 1.0) * 8).astype(np.int64)
    bits = np.where(sub, m_sub, ((e + 7) << 3) | m_norm)
    out[...] = bits.astype(np.uint8) | sign
    return out


def e4m3_decode(u) -> np.ndarray:
    """Values (fp64) of E4M3 bit patterns (NaN for S.1111.111)."""
    u = np.asarray(u, dtype=np.int64)
    s = np.where(u & 0x80, -1.0, 1.0)
    e = (u >> 3) & 15
    m = u & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def block_exponent(amax) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e (0 for amax = 0), clamped to [-127, 127].

    With amax = f * 2^E (f in [0.5, 1), math.frexp) and 448 = 0.875 * 2^9, the
    condition is f <= 0.875 * 2^(e + 9 - E), so e = E - 9 when f <= 0.875 and
    E - 8 otherwise: exact, no logarithm.
    """
    out = []
    for a in np.asarray(amax, dtype=np.float64).ravel():
        if a == 0.0:
            out.append(0)
            continue
        f, E = math.frexp(float(a))
        e = E - 9 + (1 if f > 0.875 else 0)
        out.append(min(127, max(-127, e)))
    return np.array(out, dtype=np.int64).reshape(np.shape(amax))


def quantize_blocks(x):
    """Quantise the last axis of x (length a multiple of 32) in blocks of 32.

    Returns (codes uint8 same shape, exponents int64 [..., L/32],
    dequantised fp64 same shape).
    """
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-1]
    if L % 32:
        raise ValueError("block axis must be a multiple of 32")
    xb = x.reshape(*x.shape[:-1], L // 32, 32)
    e = block_exponent(np.abs(xb).max(axis=-1))
    q = e4m3_round(xb / np.exp2(e)[..., None])
    codes = e4m3_encode(q).reshape(x.shape)
    deq = (q * np.exp2(e)[..., None]).reshape(x.shape)
    return codes, e, deq


def quantize_rows(x):
    """Q or K [..., N, d]: blocks of 32 consecutive head dims of each row.

    Returns (codes [..., N, d], exponents [..., N, d/32], dequantised).
    """
    return quantize_blocks(x)


def quantize_keys(v):
    """V [..., N, d]: blocks of 32 consecutive keys of each head dim.

    Keys are padded with zeros to a multiple of 64.  Returns (codes
    [..., d, Np] (keys contiguous), exponents [..., Np/32, d], dequantised V
    [..., N, d]).
    """
    v = np.asarray(v, dtype=np.float64)
    N = v.shape[-2]
    Np = -(-N // 64) * 64
    pad = np.zeros(v.shape[:-2] + (Np, v.shape[-1]))
    pad[..., :N, :] = v
    vt = np.swapaxes(pad, -1, -2)                       # [..., d, Np]
    codes, e, deq_t = quantize_blocks(vt)               # blocks along keys
    return codes, np.swapaxes(e, -1, -2), np.swapaxes(deq_t, -1, -2)[..., :N, :]


def attention_forward_fp8(q, k, v, scale: float, causal: bool):
    """(O, LSE, Q^, K^, V^): attention of the block-quantised inputs, fp64."""
    qd = quantize_rows(torch.as_tensor(q).double().numpy())[2]
    kd = quantize_rows(torch.as_tensor(k).double().numpy())[2]
    vd = quantize_keys(torch.as_tensor(v).double().numpy())[2]
    qd, kd, vd = (torch.from_numpy(t) for t in (qd, kd, vd))
    o, lse = attention_forward(qd, kd, vd, scale, causal)
    return o, lse, qd, kd, vd
