"""Pins of the occupancy throttle (oracle/batch.py) and of the library's
la_batch_plan against it, on the host.

"Speculative Decoding" lesson, Chapter 7 "Speculation Meets the Batch": the
step's budget of token-equivalents is shared; the batch's own rows come first
and speculation gets what is left, per request.  The pins are closed forms
for uniform requests (where the round-robin deal has one answer), the
chapter's own worked numbers restated in rows (budget 156 on its hardware;
B = 20 quiet requests each speculating k = 4 all fit; at B = 140 the 16 rows
left take at most four 4-row candidates), and the plan's defining properties
on random inputs: it fits the budget, it is maximal, it is fair turn by turn,
and pausing takes the shortest suffix.
"""
import numpy as np
import pytest

from oracle.batch import plan_rows

la = pytest.importorskip("exact_lookahead_decoding_amd.la")


def _rows(base, cap, paused, S):
    return sum((1 if p else b) + c * S for b, c, p in zip(base, cap, paused) if b > 0)


@pytest.mark.parametrize("n,b,f,S,T", [(4, 28, 7, 4, 256), (8, 28, 7, 4, 256), (5, 3, 5, 2, 30), (3, 1, 4, 6, 20),
                                       (6, 10, 2, 3, 60), (1, 60, 15, 4, 120)])
def test_uniform_requests_closed_form(n, b, f, S, T):
    assert n * b <= T
    cap, paused = plan_rows(T, S, [b] * n, [f] * n)
    total = min(n * f, (T - n * b) // S)
    q, r = divmod(total, n)
    assert cap == [q + 1] * r + [q] * (n - r)
    assert paused == [False] * n


@pytest.mark.parametrize("n,b,f,S,T", [(8, 28, 7, 4, 200), (10, 28, 7, 4, 100), (4, 60, 15, 4, 64), (3, 9, 2, 2, 4)])
def test_pause_closed_form(n, b, f, S, T):
    """Base rows over the budget: the fewest requests from the end drop their branch."""
    assert n * b > T >= n
    m = -(-(n * b - T) // (b - 1))            # smallest m with (n - m) b + m <= T
    cap, paused = plan_rows(T, S, [b] * n, [f] * n)
    assert paused == [False] * (n - m) + [True] * m
    left = T - ((n - m) * b + m)
    total = min((n - m) * f, left // S)
    q, r = divmod(total, n - m) if n > m else (0, 0)
    assert cap == [q + 1] * r + [q] * (n - m - r) + [0] * m


def test_chapter_seven_worked_numbers():
    # quiet server: 20 requests, each one ordinary row plus one 4-row candidate (k = 4 -> 5 rows); budget 156
    cap, paused = plan_rows(156, 4, [1] * 20, [1] * 20)
    assert cap == [1] * 20 and not any(paused)
    # 136 rows of headroom at B = 20 hold 34 more 4-row candidates (the chapter's "roughly 27" counts 5 per request)
    cap, _ = plan_rows(156, 4, [1] * 20, [10] * 20)
    assert sum(cap) == 136 // 4
    # near saturation: B = 140 leaves 16 rows; 30 of them wanting a 4-row candidate get four
    found = [1] * 30 + [0] * 110
    cap, paused = plan_rows(156, 4, [1] * 140, found)
    assert sum(cap) == 4 and cap[:4] == [1] * 4 and not any(paused)
    with pytest.raises(OverflowError):
        plan_rows(156, 4, [1] * 157, [0] * 157)


def _check_properties(T, S, base, found, cap, paused):
    n = len(base)
    act = [i for i in range(n) if base[i] > 0]
    rows = _rows(base, cap, paused, S)
    assert rows <= T
    for i in range(n):
        assert 0 <= cap[i] <= found[i] or (base[i] == 0 and cap[i] == 0)
        if paused[i]:
            assert base[i] > 1 and cap[i] == 0
        if base[i] == 0:
            assert cap[i] == 0 and not paused[i]
    # pausing: a suffix of the branch-carrying requests, and the shortest one that fits
    pz = [i for i in act if paused[i]]
    if pz:
        first = min(pz)
        assert all(paused[i] for i in act if i >= first and base[i] > 1)
        unpause = sum(base[i] for i in act if not paused[i]) + len(pz) - 1 + base[first]
        assert unpause > T
    # maximal: no unpaused request could take one more candidate
    if rows + S <= T:
        assert all(paused[i] or cap[i] == found[i] for i in act)
    # fair turn by turn: a request left wanting bounds everyone's count
    for i in act:
        if not paused[i] and cap[i] < found[i]:
            for j in act:
                if not paused[j]:
                    assert cap[j] <= cap[i] + (1 if j < i else 0)


@pytest.mark.parametrize("seed", range(40))
def test_plan_properties_and_library_agree(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 24))
    S = int(rng.integers(1, 8))
    base = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 70, n)]
    found = [int(x) for x in rng.integers(0, 16, n)]
    act = sum(1 for b in base if b > 0)
    T = int(rng.integers(max(act, 1), 260))
    cap, paused = plan_rows(T, S, base, found)
    _check_properties(T, S, base, found, cap, paused)
    lcap, lpaused = la.la_batch_plan(T, S, base, found)
    assert lcap == cap
    assert lpaused == [int(p) for p in paused]


def test_library_plan_rejects():
    with pytest.raises(la.LaError) as e:
        la.la_batch_plan(3, 4, [2, 2, 2, 2], [0, 0, 0, 0])
    assert e.value.code == la.LA_EOVERFLOW
    for args in [(0, 4, [1], [0]), (10, 0, [1], [0]), (10, 16, [1], [0]), (10, 4, [-1], [0]), (10, 4, [1], [-2])]:
        with pytest.raises(la.LaError) as e:
            la.la_batch_plan(*args)
        assert e.value.code == la.LA_EINVAL, args


def test_batch_bytes():
    import synthetic
    lib = la.load()
    d = la.dims_struct(synthetic.PRESETS["llama7b"])
    b1, b256 = lib.la_batch_bytes(d, 1), lib.la_batch_bytes(d, 256)
    assert 0 < b1 < b256
    assert lib.la_batch_bytes(d, 0) == 0 and lib.la_batch_bytes(d, 257) == 0
    # stacked activations and fp32 logits for 256 rows at least
    assert b256 >= 256 * 32000 * 4 + 256 * 11008 * 2
