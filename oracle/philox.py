"""Counter-based uniforms for the verify step: Philox4x64-10.

TEST INFRASTRUCTURE (see the package docstring).

Philox (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC 2011) maps a 256-bit counter and a 128-bit key to 256 random
bits through ten rounds of a bijection: per round, two 64 x 64 -> 128-bit
products of counter words with the multipliers M0, M1; the high halves are
xored with the other counter words and the round keys; the words are
permuted; the key is bumped by the Weyl constants W0, W1 between rounds.

The verify step uses one uniform per target row (reading 2: u[b, i] tests
draft i, u[b, k_b] draws the last token), on the 2^-24 grid so it is exact
in float32 (reading 1).  Slot i of request b takes word i mod 4 of the block
at counter (i div 4, b, offset, 0) under key (seed, 0), keeps its top 24 bits
and scales by 2^-24.
"""
import numpy as np

M64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(counter, key):
    """The 4 x 64-bit output block for a 4 x 64-bit counter and 2 x 64-bit key
    (Python integers)."""
    x0, x1, x2, x3 = (int(v) & M64 for v in counter)
    k0, k1 = (int(v) & M64 for v in key)
    for _ in range(10):
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> 64, p0 & M64
        hi1, lo1 = p1 >> 64, p1 & M64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & M64
        k1 = (k1 + PHILOX_W1) & M64
    return x0, x1, x2, x3


def philox_uniforms(seed: int, offset: int, B: int, slots: int) -> np.ndarray:
    """u[b, i] for b < B, i < slots, as float64 values on the 2^-24 grid."""
    u = np.empty((B, slots), dtype=np.float64)
    for b in range(B):
        for j in range((slots + 3) // 4):
            words = philox4x64_10((j, b, offset, 0), (seed, 0))
            for w in range(4):
                i = 4 * j + w
                if i < slots:
                    u[b, i] = (words[w] >> 40) * 2.0 ** -24
    return u
