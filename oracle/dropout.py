"""Attention dropout regenerated from a counter-based generator.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

[FA-WHY] §05 (fourth point): a naive implementation keeps a B x H x N x N
dropout mask for the backward pass; the fused kernel keeps only the Philox
seed and offset and regenerates the same mask in the backward pass.
[FA-CUDA] §7 adds that the random-number offset must be reproducible.

The pages do not fix the generator's variant or how its outputs map onto
(query, key) pairs.  The reading taken here:

* Generator: Philox4x64 with 10 rounds, as published by Salmon, Moraes,
  Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011):
  a 4 x 64-bit counter, a 2 x 64-bit key, and per round two 64 x 64 -> 128
  bit products with the multipliers M0, M1, the counter words permuted and
  xored with the key, and the key bumped by the Weyl constants W0, W1.
* For batch element b, query head h (bh = b*H + h), query i and key j:
  counter = (j // 16, i, bh, offset), key = (seed, 0).  The 4 output words
  hold 16 values of 16 bits; key j = 16t + e takes bits 16*(e % 4) ..
  16*(e % 4) + 15 of word e // 4.
* Key j is kept for query i iff its value >= thr = floor(p * 65536), so a
  key is dropped with probability thr / 65536 (p rounded down to a multiple
  of 2^-16); kept probabilities are scaled by 65536 / (65536 - thr), which
  keeps the expectation of the dropped P equal to P.
* The dropped P weights V in the forward pass; the LSE saved for the
  backward pass is the undropped one ([FA-WHY] §3.3 recomputes P from it).
"""

from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1


def philox4x64(counter, key, rounds=10):
    """One Philox4x64 block with Python integers: counter (4 words), key
    (2 words) -> 4 output words.  Each round: (hi0, lo0) = M0 * c0,
    (hi1, lo1) = M1 * c2, c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), then
    k0 += W0, k1 += W1 (mod 2^64)."""
    c0, c1, c2, c3 = (int(x) & _MASK64 for x in counter)
    k0, k1 = (int(x) & _MASK64 for x in key)
    for _ in range(rounds):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & _MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64)
        k0 = (k0 + PHILOX_W0) & _MASK64
        k1 = (k1 + PHILOX_W1) & _MASK64
    return [c0, c1, c2, c3]


def _mulhilo(a, m):
    """(hi, lo) of the 128-bit product of uint64 array a and constant m,
    from 32-bit limbs in uint64 arithmetic."""
    a = a.astype(np.uint64)
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    a_lo, a_hi = a & np.uint64(0xFFFFFFFF), a >> np.uint64(32)
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> np.uint64(32)) + (lh & np.uint64(0xFFFFFFFF)) + (hl & np.uint64(0xFFFFFFFF))
    lo = (ll & np.uint64(0xFFFFFFFF)) | ((mid & np.uint64(0xFFFFFFFF)) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_array(c0, c1, c2, c3, k0, k1, rounds=10):
    """The same block for arrays of counters (numpy uint64, broadcast
    together) and a scalar key; returns the 4 output words as arrays."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = np.broadcast_arrays(*(np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3)))
        k0, k1 = np.uint64(k0 & _MASK64), np.uint64(k1 & _MASK64)
        for _ in range(rounds):
            hi0, lo0 = _mulhilo(c0, PHILOX_M0)
            hi1, lo1 = _mulhilo(c2, PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0 = k0 + np.uint64(PHILOX_W0)
            k1 = k1 + np.uint64(PHILOX_W1)
    return c0, c1, c2, c3


def dropout_threshold(p):
    """thr = floor(p * 65536) for 0 <= p < 1, and the keep scale 65536 / (65536 - thr)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    thr = int(np.floor(np.float64(p) * 65536.0))
    return thr, 65536.0 / (65536 - thr)


def dropout_keep_rows(bh, N, p, seed, offset, rows=None):
    """Boolean keep mask [R, N] of head number bh (= b*H + h) for query rows
    ``rows`` (default all N), by the mapping in the module docstring."""
    thr, _ = dropout_threshold(p)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    T = -(-N // 16)
    t = np.arange(T, dtype=np.uint64)[None, :]
    i = rows.astype(np.uint64)[:, None]
    w = philox4x64_array(t, i, np.uint64(bh), np.uint64(offset), seed, 0)
    vals = np.empty((rows.size, T, 16), dtype=np.uint64)
    for e in range(16):
        vals[:, :, e] = (w[e // 4] >> np.uint64(16 * (e % 4))) & np.uint64(0xFFFF)
    return (vals >= np.uint64(thr)).reshape(rows.size, T * 16)[:, :N]


def dropout_keep(B, H, N, p, seed, offset, rows=None, heads=None):
    """Boolean keep mask [B, H, R, N] for queries ``rows`` (default all N),
    or [len(heads), R, N] for the (b, h) pairs in ``heads``.  True = kept."""
    if heads is None:
        return np.stack([dropout_keep_rows(b * H + h, N, p, seed, offset, rows)
                         for b in range(B) for h in range(H)]).reshape(B, H, -1, N)
    return np.stack([dropout_keep_rows(b * H + h, N, p, seed, offset, rows) for b, h in heads])
