"""Philox-4x32-10 counter-based generator, written from its published
definition (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3", SC 2011): a 4 x 32-bit counter and a 2 x 32-bit key; ten
rounds, each multiplying words 0 and 2 by fixed constants and mixing the
high/low halves with the other words and the key, the key bumped by the
Weyl constants between rounds.

TEST INFRASTRUCTURE ONLY (see the package docstring). The GPU sampler
implements the same generator on its side; the two share no code.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57       # round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85       # key increments (golden ratio, sqrt(3) - 1)
MASK = 0xFFFFFFFF


def philox4x32(ctr, key, rounds: int = 10):
    """Vectorised over numpy arrays: ctr is 4 uint arrays, key 2; returns 4 uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & MASK for x in ctr]
    k = [np.asarray(x, dtype=np.uint64) & MASK for x in key]
    for r in range(rounds):
        if r:
            k = [(k[0] + W0) & MASK, (k[1] + W1) & MASK]
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK)
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return [x.astype(np.uint32) for x in c]


def row_uniforms(seed: int, offset: int, row_key: int, n: int) -> np.ndarray:
    """Uniforms on (0, 1) for tokens 0..n-1 of one row, in fp64 (exact).

    Token i takes word i % 4 of Philox-4x32-10 with counter
    (i // 4, row_key low 32 bits, row_key high 32 bits, offset) and key
    (seed low 32 bits, seed high 32 bits); u = (word + 1/2) 2^-32.
    """
    blocks = (n + 3) // 4
    j = np.arange(blocks, dtype=np.uint64)
    rk = int(row_key) & 0xFFFFFFFFFFFFFFFF
    sd = int(seed) & 0xFFFFFFFFFFFFFFFF
    out = philox4x32([j, np.full(blocks, rk & MASK), np.full(blocks, rk >> 32),
                      np.full(blocks, int(offset) & MASK)],
                     [np.full(blocks, sd & MASK), np.full(blocks, sd >> 32)])
    words = np.stack(out, axis=1).reshape(-1)[:n].astype(np.float64)
    return (words + 0.5) * 2.0 ** -32
