"""Target sampling distribution and draws, in a bit-reproducible fp64 form.

The pages fix the rule (temperature warps the target distribution before
verification; "Speculative Decoding" lesson, Chapter 1; "M7.3", 0x05B) but
not its floating-point form.  Because the decisions taken here produce
integers that must agree exactly between implementations, every quantity is
defined by a fixed sequence of IEEE fp64 operations:

* a_v = (double(l_v) - double(l_max)) / T          (l = float32 logits)
* e_v = expneg(a_v)  -- Cody-Waite reduction a = k ln2 + r with the two-part
  ln2 below, p = 1 + r(1 + r/2(1 + ... (1 + r/13))) evaluated inner-first
  as p <- 1 + (r / n) * p for n = 13 .. 1, result ldexp(p, k); 0 below -745;
* sums over the vocabulary are blocked: 256 consecutive ids summed in id
  order, then the block sums added in block order;
* acceptance of a candidate token c with remaining mass m (Z minus the
  masses of tokens already rejected at this offset, subtracted in test
  order) is  u * m < e_c,  i.e. u < p(c) / (1 - sum p(rejected));
* a residual draw walks the blocked cumulative sum of e over untested
  tokens and returns the first id whose cumulative mass exceeds u * R.

(T = 1 and the true exp would give the plain softmax; this form differs
from it only by fp64 rounding.)
"""
from __future__ import annotations

import numpy as np

LN2_HI = float.fromhex("0x1.62e42fee00000p-1")
LN2_LO = float.fromhex("0x1.a39ef35793c76p-33")
INV_LN2 = float.fromhex("0x1.71547652b82fep+0")
BLOCK = 256


def expneg(a):
    a = np.asarray(a, dtype=np.float64)
    k = np.rint(a * INV_LN2)
    r = (a - k * LN2_HI) - k * LN2_LO
    p = np.ones_like(a)
    for n in range(13, 0, -1):
        p = 1.0 + (r / float(n)) * p
    out = np.ldexp(p, np.clip(k, -1100, 1100).astype(np.int64))
    return np.where(a < -745.0, 0.0, out)


def masses(logits_f32, T: float):
    """Unnormalised target masses e_v for one row of float32 logits."""
    l = np.asarray(logits_f32, dtype=np.float32).astype(np.float64)
    a = (l - l.max()) / float(T)
    return expneg(a)


def blocked_sum(e) -> float:
    total = 0.0
    for b0 in range(0, len(e), BLOCK):
        s = 0.0
        for x in e[b0:b0 + BLOCK]:
            s += float(x)
        total += s
    return total


def residual_draw(e, excluded, u: float) -> int:
    """Inverse-CDF draw over the non-excluded ids.

    Cumulative mass at id i = (block sums of earlier blocks, added in order)
    + (ids of i's block up to i, added in order); the result is the first id
    whose cumulative mass exceeds u * R, R the blocked total.  If R is 0 the
    argmax of e is returned; if rounding leaves u * R at or above every
    cumulative value, the last id with non-zero mass is returned.
    """
    w = np.array(e, dtype=np.float64)
    for t in excluded:
        w[t] = 0.0
    R = blocked_sum(w)
    if not R > 0.0:
        return int(np.flatnonzero(np.asarray(e) == np.max(e))[0])
    target = u * R
    acc = 0.0
    for b0 in range(0, len(w), BLOCK):
        local = 0.0
        for i in range(b0, min(b0 + BLOCK, len(w))):
            local += float(w[i])
            if acc + local > target:
                return i
        acc += local
    return int(np.flatnonzero(w > 0)[-1])
