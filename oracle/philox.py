"""Philox4x64-10 counter-based random numbers, written from the published algorithm.

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11 - the Philox-4x64 round function with ten
rounds: two 64x64->128-bit multiplies per round, a Weyl-sequence key schedule.

Stream layout used by tree verification (a reading; the pages only require
that rejection sampling draws r ~ Uniform(0, 1)): for node i of sequence b the
counter is (offset, b, i, 0) under key (key0, key1); of the four output words,
word 0 gives the acceptance uniform used when node i is tested as a child and
word 1 gives the resampling uniform used if the walk stops at node i.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1

# multipliers and Weyl constants of Philox-4x64 (SC'11, section 5)
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1


def _mulhilo(a: int, b: int):
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64_10(counter, key):
    """Return the 4 output words for a 4x64-bit counter and 2x64-bit key."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def node_uniforms(key, offset: int, b: int, i: int):
    """(m, K) for node i of sequence b.

    m in [1, 2^24]: the acceptance uniform is r = m / 2^24 in (0, 1].
    K in [0, 2^32): the resampling uniform is u = K / 2^32 in [0, 1).
    """
    w = philox4x64_10((offset, b, i, 0), key)
    m = (w[0] >> 40) + 1
    K = w[1] >> 32
    return m, K
