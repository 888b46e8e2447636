"""Verification: greedy survivor matching and exact one-hot sampling.

"M7.3 - Lookahead Decoding":
* 0x05A (greedy) -- the ordinary row's argmax is the first emitted token;
  candidates whose suffix disagrees with an accepted token are dropped; the
  next target token is read from the row of any survivor at that offset
  (all survivors expose the same conditional, otherwise the mask, positions
  or row map are wrong);
* 0x05B (sampling) -- at each offset the *distinct* tokens offered by the
  surviving candidates are tested in order as point masses: token c_r is
  accepted with probability p^(r-1)(c_r); a rejected token's mass is
  removed and the rest renormalised; acceptance filters the suffixes; if
  every distinct token is rejected the output is drawn from the residual.

"Speculative Decoding" lesson, Chapter 1 -- the general rule for a proposal
distribution q: accept x with min(1, p(x)/q(x)), otherwise resample from
max(0, p - q) normalised; one-hot q = delta_c reduces it to the rule above.

Readings:
* a candidate matching all S tokens emits S + 1 tokens (the extra one read
  from its last row); accepted length h lies in [0, S];
* capped convention (0x05A contrasts the paper's full match plus one target
  token with the implementation's max_hit count): with cap_full_match, at
  most S - 1 candidate tokens are accepted; the round then stops at offset
  S - 1 and emits the target token of that offset's survivor row, so it emits
  at most S tokens.  Every emitted token is still the target's;
* the winner is the lowest-index survivor (the oldest pool entry), so the
  K/V copied is that candidate's;
* sampling: greedy proposals; temperature only; draw counters
  (round, offset, k) for the k-th distinct test and (round, offset, 1024)
  for the residual/bonus draw; arithmetic as in oracle.sampling.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .numerics import argmax_lowest
from .philox import DRAW_RESIDUAL, uniform
from .sampling import blocked_sum, masses, residual_draw


def greedy_verify(out_logits, guess_logits, candidates, check_invariant=True, cap_full_match=False):
    """Survivor view.  guess_logits[c][s] is the row whose input is candidates[c][s].

    Returns (emitted, winner, h): emitted = h + 1 tokens, winner = index of the
    candidate whose rows are committed (-1 when h == 0).  With cap_full_match
    at most S - 1 offsets are matched.
    """
    S = len(candidates[0]) if candidates else 0
    target = argmax_lowest(out_logits)
    emitted = [target]
    survivors = list(range(len(candidates)))
    for offset in range(max(0, S - 1) if cap_full_match else S):
        alive = [c for c in survivors if candidates[c][offset] == target]
        if not alive:
            break
        survivors = alive
        rows = [np.asarray(guess_logits[c][offset]) for c in survivors]
        if check_invariant:
            for r in rows[1:]:
                assert np.array_equal(r, rows[0]), "survivors expose different conditionals"
        target = argmax_lowest(rows[0])
        emitted.append(target)
    h = len(emitted) - 1
    winner = survivors[0] if h > 0 else -1
    return emitted, winner, h


def greedy_hits(out_logits, guess_logits, candidates):
    """Hit-length view: hit_c = longest a with g^(c)_{1..a} = z^(c)_{1..a},
    z^(c) = (argmax out, argmax guess^(c)_1, ..., argmax guess^(c)_{S-1})."""
    hits = []
    for c, g in enumerate(candidates):
        z = [argmax_lowest(out_logits)] + [argmax_lowest(guess_logits[c][s]) for s in range(len(g) - 1)]
        a = 0
        while a < len(g) and g[a] == z[a]:
            a += 1
        hits.append(a)
    return hits


def sample_verify(out_logits, guess_logits, candidates, T: float, seed: int, round_id: int,
                  cap_full_match=False):
    """One-hot sampling verification of one round.  Returns (emitted, winner, h).
    With cap_full_match the offsets tested stop at S - 1 (the draw at offset
    S - 1 is then a plain target sample of that survivor row)."""
    S = len(candidates[0]) if candidates else 0
    last = max(0, S - 1) if cap_full_match else S      # offsets whose candidate tokens are tested
    survivors = list(range(len(candidates)))
    emitted = []
    for a in range(last + 1):
        row = out_logits if a == 0 else guess_logits[survivors[0]][a - 1]
        e = masses(row, T)
        offered = []
        if a < last:
            for c in survivors:
                t = int(candidates[c][a])
                if t not in offered:
                    offered.append(t)
        remaining = blocked_sum(e)
        rejected = []
        accepted = None
        for k, tok in enumerate(offered):
            u = uniform(seed, round_id, a, k)
            if u * remaining < e[tok]:
                accepted = tok
                break
            remaining = remaining - e[tok]
            rejected.append(tok)
        if accepted is not None:
            emitted.append(accepted)
            survivors = [c for c in survivors if candidates[c][a] == accepted]
            continue
        emitted.append(residual_draw(e, rejected, uniform(seed, round_id, a, DRAW_RESIDUAL)))
        break
    h = len(emitted) - 1
    winner = survivors[0] if h > 0 else -1
    return emitted, winner, h


def sample_token(logits, T: float, seed: int, round_id: int, offset: int = 0) -> int:
    """Plain target sample (autoregressive sampling; prefill's first token)."""
    return residual_draw(masses(logits, T), [], uniform(seed, round_id, offset, DRAW_RESIDUAL))


# ---------------------------------------------------------------------------
# exact distributions (Fractions)
# ---------------------------------------------------------------------------


def onehot_output_distribution(p: dict, offered: list) -> dict:
    """Exact output distribution at one position under the one-hot rule.

    p: token -> Fraction (sums to 1); offered: candidate tokens in test order
    (duplicates allowed; each distinct token is tested once).
    """
    out = {t: Fraction(0) for t in p}
    reach = Fraction(1)              # probability of reaching the current test
    resid = dict(p)                  # current (unnormalised) residual
    mass = Fraction(1)
    seen = []
    for t in offered:
        if t in seen:
            continue
        seen.append(t)
        acc = resid[t] / mass if mass > 0 else Fraction(0)
        out[t] += reach * acc
        reach *= (1 - acc)
        mass -= resid[t]
        resid[t] = Fraction(0)
    if mass > 0:
        for t, m in resid.items():
            out[t] += reach * m / mass
    return out


def pq_rule(p: dict, q: dict):
    """General rejection rule: accept(x) = min(1, p/q); residual prop. to max(0, p - q).

    Returns (accept probs, residual distribution, output distribution, alpha)."""
    accept = {x: (min(Fraction(1), p[x] / q[x]) if q[x] > 0 else Fraction(1)) for x in p}
    left = {x: max(Fraction(0), p[x] - q[x]) for x in p}
    z = sum(left.values())
    resid = {x: (left[x] / z if z > 0 else Fraction(0)) for x in p}
    reject_total = sum(q[x] * (1 - accept[x]) for x in p)
    output = {x: q[x] * accept[x] + reject_total * resid[x] for x in p}
    alpha = sum(min(p[x], q[x]) for x in p)
    return accept, resid, output, alpha


def naive_top1_distribution(p: dict, q: dict) -> dict:
    """Broken scheme of Chapter 1: keep a draft only if it equals the target's
    greedy top-1, otherwise emit the top-1 itself."""
    top = max(sorted(p), key=lambda x: p[x])
    out = {x: Fraction(0) for x in p}
    for x, qx in q.items():          # the draft proposes x with probability q(x)
        kept = x if x == top else top
        out[kept] += qx
    return out


def lookahead_joint(cond, prefix: tuple, candidates: list, horizon: int, cap_full_match=False) -> dict:
    """Exact joint of the first `horizon` tokens: one lookahead round with the
    given candidate suffixes (one-hot sampling verification), then plain
    autoregressive sampling.  cond(prefix) -> {token: Fraction}.  With
    cap_full_match no candidate token is offered at offset S - 1."""
    joint = {}

    def ar_tail(seq, prob):
        if len(seq) >= horizon:
            key = tuple(seq[:horizon])
            joint[key] = joint.get(key, Fraction(0)) + prob
            return
        for t, pt in cond(tuple(prefix) + tuple(seq)).items():
            if pt:
                ar_tail(seq + [t], prob * pt)

    def step(seq, survivors, a, prob):
        # seq: tokens emitted so far in this round; survivors: candidate indices
        S = len(candidates[0]) if candidates else 0
        last = max(0, S - 1) if cap_full_match else S
        p = cond(tuple(prefix) + tuple(seq))
        offered = [candidates[c][a] for c in survivors] if a < last else []
        dist_reach = Fraction(1)
        mass = Fraction(1)
        resid = dict(p)
        seen = []
        for t in offered:
            if t in seen:
                continue
            seen.append(t)
            acc = resid[t] / mass if mass > 0 else Fraction(0)
            if acc:
                nxt = [c for c in survivors if candidates[c][a] == t]
                step(seq + [t], nxt, a + 1, prob * dist_reach * acc)
            dist_reach *= (1 - acc)
            mass -= resid[t]
            resid[t] = Fraction(0)
        if mass > 0 and dist_reach:
            for t, m in resid.items():
                if m:
                    ar_tail(seq + [t], prob * dist_reach * m / mass)

    step([], list(range(len(candidates))), 0, Fraction(1))
    return joint


def ar_joint(cond, prefix: tuple, horizon: int) -> dict:
    joint = {}

    def rec(seq, prob):
        if len(seq) == horizon:
            joint[tuple(seq)] = joint.get(tuple(seq), Fraction(0)) + prob
            return
        for t, pt in cond(tuple(prefix) + tuple(seq)).items():
            if pt:
                rec(seq + [t], prob * pt)

    rec([], Fraction(1))
    return joint
