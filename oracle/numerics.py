"""Storage-precision rounding and the greedy selector.

"M7.3 - Lookahead Decoding", 0x01A (dtype ownership): hidden rows and K/V are
held in the model execution dtype, logits are promoted to float32.  The
oracle computes in fp64 and rounds to the storage dtype wherever a value is
stored.  0x02A: the greedy selector must use one fixed tie-break; ties go to
the lowest token id.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x):
    """Nearest bfloat16 value (8 significant bits, ties to even), returned as float64.

    x = m * 2**e with 0.5 <= |m| < 1 (frexp); keeping 8 significant bits means
    rounding m * 2**8 to an integer, half to even (numpy.rint).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)            # below bf16's normal range the spacing stays 2**-133
    m = x / np.ldexp(1.0, e)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    big = np.abs(r) > 3.3895313892515355e38
    if np.any(big):
        r = np.where(big, np.sign(r) * np.inf, r)
    return r


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def argmax_lowest(v) -> int:
    """Greedy selector D: index of the maximum, lowest index on ties."""
    v = np.asarray(v)
    return int(np.flatnonzero(v == v.max())[0])
