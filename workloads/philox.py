"""Philox4x32-10 counter-based generator, written from its published definition.

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11 — the Philox-4x32 bijection with 10 rounds.
One round maps the counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by the
Weyl constants (0x9E3779B9, 0xBB67AE85).  The device generator in
``workloads/csrc/wlgen.hip`` implements the same function independently; both are
checked against the published known-answer vectors in the tests.

This module holds input generation only: nothing here computes any part of the
selective scan.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Apply the 10-round Philox-4x32 bijection elementwise.

    ``c0..c3`` are uint32 arrays (broadcastable to one shape); ``k0, k1`` are the
    two 32-bit key words.  Returns four uint32 arrays.
    """
    c0 = np.asarray(c0, dtype=np.uint32)
    c1 = np.asarray(c1, dtype=np.uint32)
    c2 = np.asarray(c2, dtype=np.uint32)
    c3 = np.asarray(c3, dtype=np.uint32)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 &= 0xFFFFFFFF
    k1 &= 0xFFFFFFFF
    for _ in range(10):
        p0 = c0.astype(np.uint64) * M0
        p1 = c2.astype(np.uint64) * M1
        hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
        lo0 = (p0 & _MASK32).astype(np.uint32)
        hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
        lo1 = (p1 & _MASK32).astype(np.uint32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint32(k0), lo1,
                          hi0 ^ c3 ^ np.uint32(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return c0, c1, c2, c3


def draw_u16(key0: int, key1: int, stream: int, step: int, start: int, count: int) -> np.ndarray:
    """16-bit draws ``[start, start+count)`` of one stream.

    Element ``i`` of a stream comes from Philox block ``i // 8`` with counter
    ``(block & 0xffffffff, block >> 32, stream, step)``; the block's four 32-bit
    output words give eight 16-bit draws, low half first:
    element ``8*b + 2*w + h`` is bits ``[16h, 16h+16)`` of word ``w``.
    """
    if count <= 0:
        return np.zeros(0, dtype=np.uint16)
    b0 = start // 8
    b1 = (start + count - 1) // 8 + 1
    blocks = np.arange(b0, b1, dtype=np.uint64)
    lo = (blocks & _MASK32).astype(np.uint32)
    hi = (blocks >> np.uint64(32)).astype(np.uint32)
    w0, w1, w2, w3 = philox4x32_10(lo, hi, np.uint32(stream), np.uint32(step), key0, key1)
    words = np.stack([w0, w1, w2, w3], axis=1)                 # (nblocks, 4) uint32
    halves = np.stack([words & 0xFFFF, words >> 16], axis=2)   # (nblocks, 4, 2)
    flat = halves.reshape(-1).astype(np.uint16)
    off = start - b0 * 8
    return flat[off:off + count]
