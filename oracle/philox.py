"""Philox4x64-10 counter-based generator — test infrastructure.

Definition: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds. One round maps
counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with the paper's multipliers M0, M1; between rounds the key advances by the
Weyl constants W0 (golden ratio) and W1 (sqrt(3) - 1), each scaled to 2^64.

Use on this path (the sampling rule of Whisper-Flash §3.1 / App. A.4 needs
uniforms "keyed by (seed, request, step, position)"): key = (seed, 0),
counter = (request, step, position, stream); the uniform is the top 24 bits
of the first output word times 2^-24, exact in fp32 and fp64.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK = (1 << 64) - 1

STREAM_ACCEPT = 0
STREAM_RESAMPLE = 1
STREAM_DRAFT = 2
STREAM_DRAFT_TABLE = 3


def philox4x64_10(ctr, key):
    """Scalar reference with Python integers."""
    c0, c1, c2, c3 = (int(c) & MASK for c in ctr)
    k0, k1 = (int(k) & MASK for k in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0) & MASK, p1 & MASK, \
                         ((p0 >> 64) ^ c3 ^ k1) & MASK, p0 & MASK
    return c0, c1, c2, c3


def _mulhilo(a: int, b: np.ndarray):
    """64x64 -> 128-bit product of a constant and a uint64 array, via
    32-bit halves (numpy has no 128-bit integers)."""
    b = b.astype(np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    a_lo, a_hi = np.uint64(a & 0xFFFFFFFF), np.uint64(a >> 32)
    b_lo, b_hi = b & m32, b >> np.uint64(32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & m32) + (hl & m32)
    lo = (ll & m32) | ((mid & m32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised version over uint64 arrays (same definition)."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64)
    k1 = np.asarray(k1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = k0 + np.uint64(W0)
                k1 = k1 + np.uint64(W1)
            hi0, lo0 = _mulhilo(M0, c0)
            hi1, lo1 = _mulhilo(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform(seed: int, request: int, step: int, position: int, stream: int) -> float:
    w0 = philox4x64_10((request, step, position, stream), (seed, 0))[0]
    return (w0 >> 40) * 2.0 ** -24
