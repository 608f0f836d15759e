"""Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11).  Test infrastructure only.

Written from the paper's definition: a 4-word counter and 2-word key; each of
the 10 rounds multiplies words 0 and 2 by two fixed constants, forms the new
words from the high and low halves of the products, the key and the other two
words, and the key is bumped by two Weyl constants between rounds.

The epilogue "gumbel_max(logits / T, rng.take())" (How Pie thinks, §5
Epilogues) names a seed but no generator; this build reads it as Philox with
counter (vocab index, lane, 0, 0) and key (seed low 32 bits, seed high 32 bits).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised (broadcasting) over counters and keys; returns the four output
    words as uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK
    c1 = np.asarray(c1, dtype=np.uint64) & MASK
    c2 = np.asarray(c2, dtype=np.uint64) & MASK
    c3 = np.asarray(c3, dtype=np.uint64) & MASK
    ka = np.asarray(k0, dtype=np.uint64) & MASK
    kb = np.asarray(k1, dtype=np.uint64) & MASK
    c0, c1, c2, c3, ka, kb = np.broadcast_arrays(c0, c1, c2, c3, ka, kb)
    for r in range(10):
        if r:
            ka = (ka + np.uint64(W0)) & MASK
            kb = (kb + np.uint64(W1)) & MASK
        p0 = M0 * c0           # < 2^64, exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ ka, lo1, hi0 ^ c3 ^ kb, lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def gumbel_uniform(seed, lane, vocab_idx) -> np.ndarray:
    """u in (0,1) for vocabulary entries `vocab_idx` of readout lane `lane`:
    word 0 of Philox(counter=(v, lane, 0, 0), key=(seed lo, seed hi)), top 23
    bits, offset by half a step: u = ((x >> 9) + 0.5) * 2^-23 (exact in fp32,
    within [2^-24, 1 - 2^-24])."""
    v = np.asarray(vocab_idx, dtype=np.uint64)
    seed = np.asarray(seed, dtype=np.uint64)
    x0, _, _, _ = philox4x32_10(v, np.asarray(lane, dtype=np.uint64), 0, 0,
                                seed & MASK, seed >> np.uint64(32))
    return ((x0 >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23
