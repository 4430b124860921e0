"""Philox4x32-10 counter-based generator and the dropout keep mask — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke entry point and the benchmark's CPU-baseline leg may
import this module; the product path never does.

Why a counter-based generator: "FlashAttention 为什么不需要存下注意力矩阵" §05 (the fourth
difference between the minimal and the production kernel) notes that the kernel keeps no
dropout mask for the backward pass, only the Philox seed and offset, and regenerates the same
mask from them when it recomputes P.

Generator (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11,
the Philox-4x32 family with 10 rounds): state = four 32-bit counter words (c0, c1, c2, c3) and
two 32-bit key words (k0, k1). One round multiplies c0 by M0 and c2 by M1 as full 64-bit
products (hi:lo halves) and permutes:
    (c0, c1, c2, c3) <- (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
and between rounds the key is advanced by the Weyl constants (k0 += W0, k1 += W1, mod 2^32).
M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9 (golden ratio), W1 = 0xBB67AE85 (sqrt(3)-1).

Dropout mask (this library's definition; the pages fix only "seed + offset, regenerate"):
for head index bh = b*H + h, query i and key j,
    counter = (j // 8, i, bh, offset),  key = (seed mod 2^32, seed // 2^32)
    the four output words give eight 16-bit values, in order w0.lo, w0.hi, w1.lo, ..., w3.hi,
    for keys 8*(j//8) + 0 .. 7;  key j is kept iff its value < T,
    T = floor((1 - p) * 65536 + 1/2)  (p taken as a float32, the arithmetic in float64),
and a kept probability is multiplied by 65536 / T (so its expectation is unchanged).
"""

from __future__ import annotations

import numpy as np

__all__ = ["philox4x32", "keep_threshold", "keep_scale", "dropout_keep_ref"]

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)


def philox4x32(ctr, key, rounds=10):
    """Philox-4x32 with `rounds` rounds (10 = the published default).

    ctr: integer array [..., 4] of 32-bit words; key: (k0, k1) 32-bit words.
    Returns uint32 [..., 4].
    """
    c = np.asarray(ctr, dtype=np.uint64) & _LO
    if c.shape[-1] != 4:
        raise ValueError("counter must have 4 words in its last axis")
    c0, c1, c2, c3 = (c[..., n] for n in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for rnd in range(rounds):
        if rnd > 0:
            k0 = (k0 + W0) & _LO
            k1 = (k1 + W1) & _LO
        p0 = M0 * c0  # < 2^64: exact in uint64
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _LO,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _LO)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def keep_threshold(p):
    """T = floor((1 - p) * 65536 + 1/2) for a dropout probability p in [0, 1) (as float32)."""
    pf = float(np.float32(p))
    if not (0.0 <= pf < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor((1.0 - pf) * 65536.0 + 0.5))


def keep_scale(p):
    """Multiplier of a kept probability: 65536 / T (float64)."""
    return 65536.0 / keep_threshold(p)


def dropout_keep_ref(n_q, n_k, bh, seed, offset, p):
    """Boolean keep mask [n_q, n_k] of head index bh (= b*H + h), as defined in the module doc."""
    t = keep_threshold(p)
    groups = (n_k + 7) // 8
    ii, gg = np.meshgrid(np.arange(n_q, dtype=np.uint64), np.arange(groups, dtype=np.uint64),
                         indexing="ij")
    ctr = np.stack([gg, ii, np.full_like(ii, bh), np.full_like(ii, offset & 0xFFFFFFFF)],
                   axis=-1)
    w = philox4x32(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).astype(np.uint32)
    lo = w & np.uint32(0xFFFF)
    hi = w >> np.uint32(16)
    vals = np.stack([lo, hi], axis=-1).reshape(n_q, groups * 8)  # w0.lo, w0.hi, w1.lo, ...
    return vals[:, :n_k] < t
