"""Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), written from its
published definition.

Verifier randomness must be fresh and independent of how the candidate list
was produced ("M7.3 - Lookahead Decoding", 0x05B).  A counter-based generator
gives each decision its own draw: key = the 64-bit seed, counter =
(round, offset, draw, 0); u is the 53-bit uniform
((x0 >> 5) * 2**26 + (x1 >> 6)) * 2**-53 in [0, 1).
"""
from __future__ import annotations

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF

DRAW_RESIDUAL = 1024      # draw index of the residual / bonus / plain sample at an offset


def philox4x32_10(ctr, key):
    c = [int(x) & MASK for x in ctr]
    k0, k1 = int(key[0]) & MASK, int(key[1]) & MASK
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def uniform(seed: int, round_id: int, offset: int, draw: int) -> float:
    x = philox4x32_10([round_id, offset, draw, 0], [seed & MASK, (seed >> 32) & MASK])
    return ((x[0] >> 5) * 67108864 + (x[1] >> 6)) * (1.0 / 9007199254740992.0)
