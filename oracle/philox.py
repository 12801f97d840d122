"""Philox4x32-10, a counter-based random number generator (test infrastructure).

Written from its published definition: J. K. Salmon, M. A. Moraes, R. O. Dror
and D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011),
section 3.  The generator is a keyed bijection of a 128-bit counter: ten
rounds, each of which multiplies two of the four 32-bit counter words by fixed
odd constants, keeps the low halves of the two 64-bit products and mixes their
high halves into the other two words together with the round key; the 64-bit
key is advanced between rounds by two Weyl increments (the leading bits of the
golden ratio and of sqrt(3) - 1).  Output = the four words after round ten.

The dropout of attention draws its random numbers from this generator (the
forward keeps only the generator's key and regenerates the mask in the
backward: "FlashAttention and GPU memory", section 09; "Lecture 8 . GPU
Performance & FlashAttention", section 5.4).

Pinned in tests against an independent implementation (rocRAND's), and the
Weyl increments against their closed forms.  Only ``tests/``,
``__graft_entry__.smoke()`` and bench's cpu_baseline use it.
"""
from __future__ import annotations

import numpy as np

__all__ = ["MULT", "WEYL", "philox4x32_10"]

MULT = (0xD2511F53, 0xCD9E8D57)   # round multipliers of words 0 and 2
WEYL = (0x9E3779B9, 0xBB67AE85)   # key increments between rounds
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 of counters [..., 4] under keys [..., 2] (uint32).

    Broadcasts counter against key; returns uint32 [..., 4].  One round maps
    (x0, x1, x2, x3) with round key (k0, k1) to
        (hi(M1 x2) ^ x1 ^ k0,  lo(M1 x2),  hi(M0 x0) ^ x3 ^ k1,  lo(M0 x0)),
    and the key gains (W0, W1) before each of rounds 2..10.
    """
    ctr = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    x0, x1, x2, x3 = (ctr[..., i] & _M32 for i in range(4))
    k0, k1 = k[..., 0] & _M32, k[..., 1] & _M32
    m0, m1 = np.uint64(MULT[0]), np.uint64(MULT[1])
    w0, w1 = np.uint64(WEYL[0]), np.uint64(WEYL[1])
    for rnd in range(10):
        if rnd:
            k0 = (k0 + w0) & _M32
            k1 = (k1 + w1) & _M32
        p0 = m0 * x0          # < 2^64: both factors are below 2^32
        p1 = m1 * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & _M32,
                          (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & _M32)
    return np.stack(np.broadcast_arrays(x0, x1, x2, x3), axis=-1).astype(np.uint32)
