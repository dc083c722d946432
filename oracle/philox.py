"""Philox4x64-10 in numpy (oracle; test infrastructure only).

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11, section on the Philox family.
A 256-bit counter (four 64-bit words) and a 128-bit key (two words) go through
ten rounds.  Each round multiplies words 0 and 2 by two fixed odd constants
into 128-bit products; the new state is
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0)),
and between rounds the key is advanced by two Weyl constants.

The stochastic-rounding stream of the bf16 weight write-back (FORGE explainer,
Technical Summary section 2 "Precision and Fidelity": stochastic rounding of
weight write-backs) draws 16 bits per weight element from this generator; see
numerics.sr_bits for the element -> (counter, key, bit field) map.

Pinned against numpy.random.Philox (the same generator, a library routine).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B

_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def mulhilo64(a: np.ndarray, b: int):
    """Full 128-bit product of uint64 array a and constant b -> (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    bl, bh = np.uint64(b & 0xFFFFFFFF), np.uint64(b >> 32)
    al, ah = a & _M32, a >> _S32
    ll, lh, hl, hh = al * bl, al * bh, ah * bl, ah * bh
    mid = (ll >> _S32) + (lh & _M32) + (hl & _M32)
    lo = (ll & _M32) | ((mid & _M32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x64 rounds on broadcastable uint64 arrays; returns four words."""
    c = [np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3)]
    k = [np.asarray(k0, dtype=np.uint64), np.asarray(k1, dtype=np.uint64)]
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k = [k[0] + np.uint64(W0), k[1] + np.uint64(W1)]
            hi0, lo0 = mulhilo64(c[0], M0)
            hi1, lo1 = mulhilo64(c[2], M1)
            c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return c
