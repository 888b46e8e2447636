"""Batched rounds (la_batch_step) on the GPU through the C ABI.

"Speculative Decoding" lesson, Chapter 7 "Speculation Meets the Batch": the
requests of a step share one read of the weights, and speculation spends only
the rows their own rounds leave in the step's budget, throttled per request.

* tiny fp32 decoder, five requests of one N with different W / G, one
  autoregressive and one sampled, under a budget that pauses and caps them:
  every step's per-request candidates found / verified, pause, accepted
  length and emitted tokens equal the oracle's batch (oracle/batch.py); the
  final outputs, windows and pools equal the oracle's, and the greedy
  outputs equal autoregressive greedy;
* with a budget that throttles nothing, each request's rounds are those of
  its own la_step, bit for bit (tiny fp32 and small bf16 GQA); again with
  prompts long enough that every request's keys are cut in several splits,
  on small bf16, on a two-layer model of 7B's shape (32 heads of 128) and
  on a two-layer model of CodeLlama-34B's shape (64 query heads on 8 KV
  heads), which run the per-request passes as one launch per layer with
  requests of different key splits and capacities side by side;
* a throttled bf16 batch still emits the GPU autoregressive tokens;
* bad batches are refused before anything runs.
"""
import numpy as np
import pytest

import synthetic
from oracle.batch import batch_generate
from oracle.decode import ar_generate
from oracle.model import OracleModel
from oracle import pool as opool

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
la = pytest.importorskip("exact_lookahead_decoding_amd.la")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _model(name, seed=0):
    dims = synthetic.PRESETS[name]
    w = synthetic.model_weights(dims, seed)
    return dims, w, la.DeviceModel(dims, weights=w), OracleModel(dims, w)


@pytest.fixture(scope="module")
def tiny():
    return _model("tiny")


@pytest.fixture(scope="module")
def small_bf16():
    return _model("small_bf16")


def _specs(vocab):
    mk = synthetic.markov_prompt
    return [
        dict(prompt=mk(vocab, 32, 0), W=5, N=4, G=5, max_new=48),
        dict(prompt=mk(vocab, 40, 1), W=4, N=4, G=3, max_new=40),
        dict(prompt=synthetic.copyspan_prompt(vocab, 80, 2)[0], W=6, N=4, G=6, max_new=56, pool_from_output=True),
        dict(prompt=mk(vocab, 28, 3), W=5, N=4, G=5, max_new=30, ar_only=True),
        dict(prompt=mk(vocab, 36, 4), W=5, N=4, G=5, max_new=40, mode="sample", T=0.7, seed=5),
    ]


def _session(dm, spec):
    kw = dict(W=spec["W"], N=spec["N"], G=spec["G"], max_new=spec["max_new"], ar_only=spec.get("ar_only", False),
              max_prompt=spec.get("max_prompt"), pool_from_output=spec.get("pool_from_output", False))
    if spec.get("mode") == "sample":
        kw.update(verify_mode=la.LA_VERIFY_SAMPLE, temperature=spec["T"], seed=spec["seed"])
    return la.Session(dm, spec["prompt"], **kw)


def _run_batch(batch, sessions, budget):
    steps = []
    while True:
        toks, info = batch.la_batch_step(sessions, row_budget=budget)
        if all(i.Q == 0 for i in info):
            return steps
        steps.append((toks, info))
        assert sum(i.Q for i in info) <= (budget or batch.max_rows)


@pytest.mark.parametrize("budget", [40, 24])
def test_tiny_throttled_batch_matches_oracle(tiny, budget):
    dims, w, dm, om = tiny
    specs = _specs(dims.vocab)
    reqs, ref = batch_generate(om, specs, budget)
    sessions = [_session(dm, s) for s in specs]
    batch = la.Batch(dm, max_rows=64)
    got = _run_batch(batch, sessions, budget)
    assert len(got) == len(ref)
    n_paused = n_capped = 0
    for t, ((toks, info), rstep) in enumerate(zip(got, ref)):
        for i, (tk, inf, rr) in enumerate(zip(toks, info, rstep)):
            if rr is None:
                assert inf.Q == 0 and tk == [], (t, i)
                continue
            print(f"step {t} req {i}: Q={inf.Q} found={inf.found} verified={inf.verified} paused={inf.paused} "
                  f"h={inf.h}", flush=True)
            assert (inf.found, inf.verified, bool(inf.paused), inf.h) == \
                (rr["found"], rr["verified"], rr["paused"], rr["h"]), (t, i)
            n_paused += inf.paused
            n_capped += inf.verified < inf.found
            left = specs[i]["max_new"] - sum(len(g[0][i]) for g in got[:t]) - 1
            assert tk == rr["emitted"][:left], (t, i)
    assert n_paused > 0 and n_capped > 0            # the throttle is exercised both ways
    for i, (s, r, spec) in enumerate(zip(sessions, reqs, specs)):
        st = s.la_get_state()
        assert st["output"] == r.out, i
        if spec.get("mode") != "sample":
            assert r.out == ar_generate(om, spec["prompt"], spec["max_new"]), i
        if not spec.get("ar_only"):
            assert st["levels"] == r.window, i
            for key in range(dims.vocab):
                assert s.la_pool_lookup(key) == opool.lookup(r.token_map, key, spec["G"]), (i, key)
        assert s.la_stats()["paused"] == sum(1 for rec in r.rounds if rec.paused), i


def _single_rounds(dm, spec):
    s = _session(dm, spec)
    rounds = []
    while True:
        t = s.la_step()
        if not t:
            return s, rounds
        rounds.append(t)


@pytest.mark.parametrize("name", ["tiny", "small_bf16"])
def test_unthrottled_batch_equals_single_sessions(tiny, small_bf16, name):
    dims, w, dm, om = tiny if name == "tiny" else small_bf16
    specs = _specs(dims.vocab)
    singles = [_single_rounds(dm, s) for s in specs]
    sessions = [_session(dm, s) for s in specs]
    batch = la.Batch(dm, max_rows=256)
    got = _run_batch(batch, sessions, 0)
    for i, (s_one, rounds) in enumerate(singles):
        mine = [toks[i] for toks, info in got if info[i].Q > 0]
        assert mine == rounds, i
        a, b = s_one.la_get_state(), sessions[i].la_get_state()
        assert a == b, i
        sa, sb = s_one.la_stats(), sessions[i].la_stats()
        assert sa == sb and sb["paused"] == 0, i
        if not specs[i].get("ar_only"):
            for key in range(dims.vocab):
                assert s_one.la_pool_lookup(key) == sessions[i].la_pool_lookup(key), (i, key)


def _long_specs(vocab):
    mk = synthetic.markov_prompt
    return [
        dict(prompt=mk(vocab, 300, 10), W=5, N=4, G=5, max_new=24),
        dict(prompt=mk(vocab, 140, 11), W=4, N=4, G=3, max_new=20, max_prompt=900),
        dict(prompt=synthetic.copyspan_prompt(vocab, 520, 12)[0], W=6, N=4, G=6, max_new=28),
        dict(prompt=mk(vocab, 40, 13), W=5, N=4, G=5, max_new=16, ar_only=True),
        dict(prompt=mk(vocab, 200, 14), W=5, N=4, G=5, max_new=20, mode="sample", T=0.8, seed=3),
    ]


@pytest.fixture(scope="module")
def l7_2l():
    dims = synthetic.PRESETS["llama7b_2l"]
    return dims, la.DeviceModel(dims, seed=0)


@pytest.fixture(scope="module")
def cl34_2l():
    # CodeLlama-34B widths at two layers (GQA: 64 query heads on 8 KV heads)
    dims = synthetic.ModelDims(2, 8192, 64, 8, 128, 22016, 32000, "bf16")
    return dims, la.DeviceModel(dims, seed=0)


@pytest.mark.parametrize("name", ["small_bf16", "llama7b_2l", "codellama34b_2l"])
def test_long_unthrottled_batch_equals_single_sessions(request, name):
    if name == "small_bf16":
        sb = request.getfixturevalue("small_bf16")
        dims, dm = sb[0], sb[2]
    else:
        dims, dm = request.getfixturevalue("l7_2l" if name == "llama7b_2l" else "cl34_2l")
    specs = _long_specs(dims.vocab)
    singles = [_single_rounds(dm, s) for s in specs]
    sessions = [_session(dm, s) for s in specs]
    batch = la.Batch(dm, max_rows=256)
    got = _run_batch(batch, sessions, 0)
    for i, (s_one, rounds) in enumerate(singles):
        print(f"request {i}: {len(rounds)} rounds", flush=True)
        mine = [toks[i] for toks, info in got if info[i].Q > 0]
        assert mine == rounds, i
        assert s_one.la_get_state() == sessions[i].la_get_state(), i
        assert s_one.la_stats() == sessions[i].la_stats(), i


def test_bf16_throttled_batch_equals_ar(small_bf16):
    dims, w, dm, om = small_bf16
    specs = [s for s in _specs(dims.vocab) if s.get("mode") != "sample"]
    sessions = [_session(dm, s) for s in specs]
    batch = la.Batch(dm, max_rows=32)
    got = _run_batch(batch, sessions, 30)
    assert any(inf.paused for _, info in got for inf in info)
    for i, spec in enumerate(specs):
        ar = _session(dm, dict(spec, ar_only=True)).la_generate()
        assert sessions[i].la_get_state()["output"] == ar, i


def test_batch_refusals_change_nothing(tiny):
    dims, w, dm, om = tiny
    specs = _specs(dims.vocab)[:3]
    sessions = [_session(dm, s) for s in specs]
    batch = la.Batch(dm, max_rows=32)
    before = [s.la_get_state() for s in sessions]

    def refused(code, sess, budget=0, b=batch):
        with pytest.raises(la.LaError) as e:
            b.la_batch_step(sess, row_budget=budget)
        assert e.value.code == code

    refused(la.LA_EINVAL, sessions, budget=33)                     # budget above max_rows
    refused(la.LA_EINVAL, [sessions[0], sessions[1], sessions[0]])  # a request twice
    other = la.DeviceModel(dims, weights=synthetic.model_weights(dims, 1))
    refused(la.LA_EINVAL, sessions + [_session(other, specs[0])])    # another model
    refused(la.LA_EINVAL, sessions + [_session(dm, dict(specs[0], N=3))])   # another N
    refused(la.LA_EOVERFLOW, sessions, budget=2)                   # fewer rows than requests
    assert [s.la_get_state() for s in sessions] == before
    # and the same requests still decode to autoregressive greedy afterwards
    _run_batch(batch, sessions, 0)
    for s, spec in zip(sessions, specs):
        assert s.la_get_state()["output"] == ar_generate(om, spec["prompt"], spec["max_new"])
