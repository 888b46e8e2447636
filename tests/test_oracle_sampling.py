"""Sampled verification: exact enumeration, Monte Carlo against the target, and the sampler's arithmetic."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import philox, sampling, verify


def test_expneg_matches_exp():
    a = -np.concatenate([np.linspace(0, 745, 20001), np.random.default_rng(0).exponential(5, 5000)])
    a = a[a >= -745]
    got = sampling.expneg(a)
    want = np.exp(a)
    rel = np.abs(got - want) / np.maximum(want, 1e-300)
    assert np.max(rel[want > 1e-300]) < 4e-16
    assert sampling.expneg(np.array([0.0]))[0] == 1.0
    assert sampling.expneg(np.array([-800.0]))[0] == 0.0


def test_blocked_sum_and_residual_draw_grid():
    rng = np.random.default_rng(1)
    e = rng.random(700)
    e[::7] = 0.0
    assert sampling.blocked_sum(e) == pytest.approx(e.sum(), rel=1e-13)
    excluded = [3, 10, 600]
    w = e.copy()
    w[excluded] = 0
    p = w / w.sum()
    n = 20000
    counts = np.zeros(700)
    for i in range(n):
        counts[sampling.residual_draw(e, excluded, (i + 0.5) / n)] += 1
    assert counts[excluded].sum() == 0 and counts[e == 0].sum() == 0
    assert np.max(np.abs(counts / n - p)) <= 1.0 / n + 1e-12   # a u-grid hits each token's CDF interval


def _random_cond(V, seed):
    rng = np.random.default_rng(seed)
    cache = {}

    def cond(prefix):
        if prefix not in cache:
            w = rng.integers(0, 6, V)
            w[rng.integers(V)] += 1
            tot = int(w.sum())
            cache[prefix] = {t: Fraction(int(w[t]), tot) for t in range(V)}
        return cache[prefix]
    return cond


@pytest.mark.parametrize("case", range(12))
def test_lookahead_sampling_joint_equals_ar_joint(case):
    rng = np.random.default_rng(100 + case)
    V = 3 + case % 2
    S = 1 + case % 3
    C = 1 + case % 4
    cond = _random_cond(V, case)
    base = [tuple(int(t) for t in rng.integers(0, V, S)) for _ in range(C)]
    # shared prefixes and duplicates on purpose
    cands = base + [base[0][:1] + tuple(int(t) for t in rng.integers(0, V, S - 1))] + [base[-1]]
    horizon = S + 2
    assert verify.lookahead_joint(cond, (0,), cands, horizon) == verify.ar_joint(cond, (0,), horizon)


@pytest.mark.parametrize("case", range(6))
def test_capped_sampling_joint_equals_ar_joint(case):
    """The capped full-match convention (no candidate token tested at offset
    S - 1; that position is a plain target draw) is exact as well."""
    rng = np.random.default_rng(300 + case)
    V = 3 + case % 2
    S = 2 + case % 2
    C = 1 + case % 3
    cond = _random_cond(V, 50 + case)
    base = [tuple(int(t) for t in rng.integers(0, V, S)) for _ in range(C)]
    cands = base + [base[0]]
    horizon = S + 2
    capped = verify.lookahead_joint(cond, (0,), cands, horizon, cap_full_match=True)
    assert capped == verify.ar_joint(cond, (0,), horizon)


def test_naive_greedy_check_is_not_exact():
    """Keeping a candidate only when it equals the greedy top-1 collapses the distribution."""
    V = 3
    cond = _random_cond(V, 5)
    p = cond((0,))
    top = max(range(V), key=lambda t: (p[t], -t))
    naive = {t: Fraction(int(t == top)) for t in range(V)}
    exact = verify.onehot_output_distribution(p, [top])
    assert exact == p and naive != p


def test_onehot_distribution_duplicates():
    p = {0: Fraction(1, 2), 1: Fraction(1, 4), 2: Fraction(1, 8), 3: Fraction(1, 8)}
    assert verify.onehot_output_distribution(p, [1, 1, 0, 1, 2]) == p
    assert verify.onehot_output_distribution(p, []) == p
    # removing a duplicate's mass twice (no dedup) breaks exactness ("M7.3", 0x05B)
    reach, mass, resid = Fraction(1), Fraction(1), dict(p)
    out = {t: Fraction(0) for t in p}
    for t in [1, 1]:
        acc = resid[t] / mass
        out[t] += reach * acc
        reach *= 1 - acc
        mass -= p[t]
        resid[t] = Fraction(0)
    for t, m in resid.items():
        out[t] += reach * m / mass
    assert out != p


def test_sample_verify_monte_carlo_first_token():
    """Empirical distribution of the first emitted token equals the target p (4 sigma)."""
    V = 6
    logits = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.0], np.float32)
    T = 0.7
    e = sampling.masses(logits, T)
    p = e / e.sum()
    cands = [(3, 1), (3, 2), (1, 0), (5, 5), (3, 4)]
    guess = [[np.zeros(V, np.float32)] * 2 for _ in cands]
    n = 6000
    counts = np.zeros(V)
    for r in range(n):
        em, win, h = verify.sample_verify(logits, guess, cands, T, seed=42, round_id=r + 1)
        counts[em[0]] += 1
        if h:
            assert cands[win][:h] == tuple(em[:h])
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(counts / n - p) < 4 * sigma + 1e-9)


def test_sample_verify_offsets_and_bonus():
    """Certain acceptance walks all S offsets and draws a bonus from the last survivor row."""
    V, S = 5, 3
    big = np.float32(80.0)

    def onehot(t):
        r = np.full(V, -big, np.float32)
        r[t] = big
        return r
    cands = [(2, 0, 1), (2, 4, 4), (2, 4, 3)]
    guess = [[onehot(c[s + 1]) if s + 1 < S else onehot(1) for s in range(S)] for c in cands]
    guess[1][S - 1] = onehot(0)
    out = onehot(2)
    em, win, h = verify.sample_verify(out, guess, cands, 1.0, seed=3, round_id=9)
    # offset 0 accepts 2 (all survive); offset 1 row = candidate 0's -> 0 accepted
    assert em == [2, 0, 1, 1] and h == 3 and win == 0


def test_sample_verify_capped_stops_before_last_offset():
    """Under cap_full_match the same certain acceptances stop after S - 1
    offsets: the S-th token is a plain draw from the survivor's row at offset
    S - 2 (a one-hot row, so it is that row's token), h = S - 1."""
    V, S = 5, 3
    big = np.float32(80.0)

    def onehot(t):
        r = np.full(V, -big, np.float32)
        r[t] = big
        return r
    cands = [(2, 0, 1), (2, 4, 4), (2, 4, 3)]
    guess = [[onehot(c[s + 1]) if s + 1 < S else onehot(1) for s in range(S)] for c in cands]
    em, win, h = verify.sample_verify(onehot(2), guess, cands, 1.0, seed=3, round_id=9, cap_full_match=True)
    assert em == [2, 0, 1] and h == 2 and win == 0


def test_uniform_is_53_bit():
    u = philox.uniform(123456789012345, 5, 2, 1)
    assert 0.0 <= u < 1.0 and u * 2 ** 53 == int(u * 2 ** 53)
