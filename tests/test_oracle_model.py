"""The oracle's model and round machine against identities that do not depend on it.

The pages print no activations, so the forward is pinned by textbook
identities and by the equalities the method guarantees: separate forwards
== dense mask (tier 1 == tier 2), lookahead greedy == autoregressive greedy,
and pool == the trajectory n-grams.
"""
import math

import numpy as np
import pytest

import synthetic
from oracle import attention, numerics, pool, rows
from oracle.decode import ar_generate, lookahead_generate
from oracle.model import OracleModel


@pytest.fixture(scope="module")
def tiny():
    dims = synthetic.PRESETS["tiny"]
    return OracleModel(dims, synthetic.model_weights(dims, 0))


@pytest.fixture(scope="module")
def small_bf16():
    dims = synthetic.PRESETS["small_bf16"]
    return OracleModel(dims, synthetic.model_weights(dims, 0))


def test_round_bf16_against_bit_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    via_bits = synthetic.f32_from_bf16_bits(synthetic.bf16_bits_from_f32(x)).astype(np.float64)
    assert np.array_equal(numerics.round_bf16(x.astype(np.float64)), via_bits)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert numerics.round_bf16(1 + 2 ** -8) == 1.0
    assert numerics.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert numerics.round_bf16(0.0) == 0.0
    assert numerics.argmax_lowest([1, 3, 3, 2]) == 1


def _explicit_attention(q, kp, vp, kn, vn, vis):
    Qn, H, dh = q.shape
    Hkv, T, _ = kp.shape
    out = np.zeros((Qn, H, dh))
    for i in range(Qn):
        for h in range(H):
            g = h // (H // Hkv)
            keys = [kp[g, t] for t in range(T)] + [kn[j, g] for j in range(Qn) if vis[i, j]]
            vals = [vp[g, t] for t in range(T)] + [vn[j, g] for j in range(Qn) if vis[i, j]]
            sc = [sum(float(a) * float(b) for a, b in zip(q[i, h], k)) / math.sqrt(dh) for k in keys]
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            z = sum(w)
            for d in range(dh):
                out[i, h, d] = sum(wi * float(v[d]) for wi, v in zip(w, vals)) / z
    return out


def test_lookahead_attention_definition():
    c = rows.compile_round(5, 9, [[1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]], [(1, 2, 3), (4, 5, 6)], 3)
    q, kp, vp, kn, vn = synthetic.attention_op_inputs(c.Q, 4, 2, 8, 9, seed=1, dtype="f32")
    got = attention.lookahead_attention(q, kp, vp, kn, vn, c.visible)
    want = _explicit_attention(q, kp, vp, kn, vn, c.visible)
    assert np.allclose(got, want, atol=1e-12, rtol=0)


def test_rope_and_rmsnorm_identities(tiny):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 16))
    k = rng.standard_normal((1, 2, 16))
    for p0, p1, d in [(3, 7, 11), (0, 50, 5)]:
        a = np.sum(tiny.rope(q, [p0]) * tiny.rope(k, [p1]))
        b = np.sum(tiny.rope(q, [p0 + d]) * tiny.rope(k, [p1 + d]))
        assert a == pytest.approx(b, abs=1e-12)                # relative-position property
    assert np.allclose(np.linalg.norm(tiny.rope(q, [123]), axis=-1), np.linalg.norm(q, axis=-1))
    assert np.array_equal(tiny.rope(q, [0]), q)
    x = rng.standard_normal((3, 64))
    w = np.ones(64)
    assert np.allclose(tiny.rms_norm(x, w), tiny.rms_norm(4.0 * x, w), atol=1e-6)


def test_tier1_equals_tier2_logits(tiny):
    prompt = synthetic.markov_prompt(256, 32, 0)
    cache, _ = tiny.prefill(prompt)
    comp = rows.compile_round(17, cache.length, [[3, 4, 5, 6, 7], [8, 9, 10, 11, 12]], [(1, 2), (3, 4), (1, 5)], 2)
    lg2, _, _ = tiny.forward(comp.tokens, comp.positions, cache, comp.visible)
    for i, r in enumerate(comp.rows):
        vis = sorted((j for j in range(comp.Q) if comp.visible[i, j]), key=lambda j: comp.rows[j].logical_position)
        seq = list(prompt) + [comp.rows[j].token for j in vis]
        assert np.allclose(tiny.sequence_logits(seq), lg2[i], atol=1e-9, rtol=0)


@pytest.mark.parametrize("W,N,G", [(5, 3, 5), (4, 4, 3), (3, 5, 2), (6, 3, 1)])
def test_lookahead_greedy_equals_ar_tiny(tiny, W, N, G):
    prompt = synthetic.markov_prompt(256, 32, 0)
    ar = ar_generate(tiny, prompt, 64)
    la = lookahead_generate(tiny, prompt, W, N, G, 64)
    assert la["tokens"] == ar
    assert len(la["rounds"]) < 63                                  # some acceptance happened
    # warmup: N-2 rounds without candidates, then the ragged steady layout
    for r in la["rounds"][: N - 2]:
        assert r.candidates == [] and r.h == 0
    for r in la["rounds"][N - 2:]:
        assert r.level_sizes == [W - 1] + [W] * (N - 2)


def test_lookahead_greedy_equals_ar_bf16(small_bf16):
    prompt = synthetic.markov_prompt(1024, 40, 1)
    ar = ar_generate(small_bf16, prompt, 40)
    la = lookahead_generate(small_bf16, prompt, 4, 4, 4, 40)
    assert la["tokens"] == ar


def test_tier1_lookahead_equals_ar(tiny):
    prompt = synthetic.markov_prompt(256, 32, 0)
    la = lookahead_generate(tiny, prompt, 4, 4, 3, 30, tier=1)
    assert la["tokens"] == ar_generate(tiny, prompt, 30)


def test_pool_is_exactly_the_trajectory_ngrams(tiny):
    W, N, G = 5, 4, 3
    prompt = synthetic.markov_prompt(256, 32, 0)
    la = lookahead_generate(tiny, prompt, W, N, G, 64)
    replay = {}
    for r in la["rounds"]:
        if None in r.level_sizes:
            continue
        # each deepest-level row's visible path ends with the N-1 tokens before
        # its output; that output closes one n-gram per window column
        for col, path, zj in zip(r.inp_columns, r.deep_paths, r.z):
            gram = path[-(N - 1):] + [zj]
            pool.lru_upsert(replay, gram[0], tuple(gram[1:]), G)
    assert replay == la["token_map"]
    assert all(len(v) <= G for v in replay.values())


def test_generated_prefix_insertion_keeps_ar_and_pool(tiny):
    """With the generated-prefix insertion the output is still autoregressive
    greedy, and the pool is the replay of the trajectory n-grams of each round
    followed by the n-grams that round's new tokens complete (the first token's
    at the start), with the same lookups feeding later rounds."""
    W, N, G = 5, 4, 3
    prompt = synthetic.markov_prompt(256, 32, 0)
    la = lookahead_generate(tiny, prompt, W, N, G, 64, pool_from_output=True)
    assert la["tokens"] == ar_generate(tiny, prompt, 64)
    replay = {}
    seq = list(prompt) + la["tokens"][:1]
    pool.insert_output_ngrams(replay, seq, len(prompt), len(seq), N, G)
    for r in la["rounds"]:
        if None not in r.level_sizes:
            for col, path, zj in zip(r.inp_columns, r.deep_paths, r.z):
                gram = path[-(N - 1):] + [zj]
                pool.lru_upsert(replay, gram[0], tuple(gram[1:]), G)
        n0 = len(seq)
        seq += r.emitted[: 64 - (len(seq) - len(prompt))]
        pool.insert_output_ngrams(replay, seq, n0, len(seq), N, G)
    assert seq == list(prompt) + la["tokens"]
    assert replay == la["token_map"]
    # the insertion changes what later rounds look up: not the plain run's rounds
    plain = lookahead_generate(tiny, prompt, W, N, G, 64)
    assert [r.candidates for r in plain["rounds"]] != [r.candidates for r in la["rounds"]]
