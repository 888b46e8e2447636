"""Several requests decoded together, with the occupancy throttle -- TEST INFRASTRUCTURE ONLY.

"Speculative Decoding" lesson, Chapter 7 "Speculation Meets the Batch":
concurrent requests share one read of the weights per step, and the
compute a step can spend before it stops being memory-bound is a fixed
budget of token-equivalents of which the batch's own rows claim their share
first; speculation may spend only what is left, and a scheduler throttles it
per request ("Per-request adaptivity"), down to switching it off.  For
lookahead decoding the cost of a round is its packed row count (the section
on why the budget does not hit every technique alike: lookahead folds its
drafting into the verification pass, so its whole cost is its rows).  "M7.3",
0x03B: every request keeps its own pool (no global pool budget), window and
K/V.

Readings taken here (the chapter leaves the policy table and the fairness
rule open):
* the budget is counted in packed rows per step;
* every request keeps its ordinary row and, while the budget allows, its
  lookahead branch; when the requests' own rows exceed the budget, the
  requests from the last one backwards run without their lookahead branch
  (a paused round: one row, no candidates, pool and window unchanged) until
  the rest fits -- request order is the priority order the chapter leaves to
  the operator;
* the requests of one batch share N, so a candidate costs the same S rows
  in every request;
* what is left is dealt in whole candidates (S rows each), one per request
  in turn, in request order, to requests that kept their branch, up to the
  candidates each request's lookup returned.

Parity status: plan_rows is pinned by closed forms (uniform requests) and by
its defining properties on random inputs in tests/test_oracle_batch.py; the
rounds are decode.LookaheadRequest's, which is pinned by the single-request
tests.
"""
from __future__ import annotations

from .decode import LookaheadRequest


def plan_rows(budget: int, S: int, base, found):
    """The plan of one step: returns (cap, paused) per request.

    base[i]: rows of request i's round without candidates (0: not in the
    step); found[i]: candidates its lookup returned.  Raises OverflowError if
    the active requests alone exceed the budget (one row each)."""
    n = len(base)
    active = [i for i in range(n) if base[i] > 0]
    if len(active) > budget:
        raise OverflowError(f"{len(active)} requests > budget {budget}")

    def rows_with(paused_from):
        # rows when every request at index >= paused_from that has a branch drops it
        return sum((1 if (i >= paused_from and base[i] > 1) else base[i]) for i in active)

    # the largest suffix start whose pausing makes the base rows fit
    start = n
    while rows_with(start) > budget:
        start -= 1
    paused = [i >= start and base[i] > 1 for i in range(n)]
    left = budget - rows_with(start)
    blocks = left // S
    # candidate blocks in (turn k, request i) order among requests that kept their branch
    order = sorted((k, i) for i in active if not paused[i] for k in range(found[i]))
    cap = [0] * n
    for k, i in order[:blocks]:
        cap[i] += 1
    return cap, paused


def batch_generate(model, specs, budget: int):
    """Run the requests described by specs (dicts of LookaheadRequest
    arguments: prompt, W, N, G, max_new, optional mode / T / seed / ar_only
    ...) together until all are done.  Each step plans the rows of every
    unfinished request with plan_rows and runs one round of each.  Returns
    (requests, steps): steps[t] lists, per request, None if it was done, else
    dict(found, verified, paused, h, emitted)."""
    reqs = [LookaheadRequest(model, **spec) for spec in specs]
    S = {r.S for r in reqs}
    assert len(S) == 1, "the requests of one batch share N (one candidate block size)"
    s_blk = S.pop()
    steps = []
    while not all(r.done() for r in reqs):
        base = [0 if r.done() else r.base_rows() for r in reqs]
        cands = [[] if r.done() else r.candidates() for r in reqs]
        found = [len(c) for c in cands]
        cap, paused = plan_rows(budget, s_blk, base, found)
        step = []
        for i, r in enumerate(reqs):
            if r.done():
                step.append(None)
                continue
            rec = r.round(cap=cap[i], paused=paused[i])
            step.append(dict(found=found[i], verified=len(rec.candidates), paused=paused[i], h=rec.h,
                             emitted=list(rec.emitted)))
        steps.append(step)
    return reqs, steps
