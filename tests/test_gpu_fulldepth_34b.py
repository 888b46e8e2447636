"""GPU tests at the 34B shape's full depth and size, through the C ABI.

CodeLlama-34B shape (48 layers, d 8192, 64 query heads on 8 KV heads, MLP
22016, vocab 32000, bf16), 2048-token copy-span prompt, W=15 N=7 G=15: 20
lookahead rounds (up to 180 packed rows) emit exactly the tokens of GPU
autoregressive decoding with the same kernels ("M7.3" 0x02A; the kernels are
batch invariant, so the bits agree), with the pool empty at the start and
seeded with the prompt's n-grams.
"""
import pytest

import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
la = pytest.importorskip("exact_lookahead_decoding_amd.la")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _say(*a):
    print(*a, flush=True)


def _lookahead_vs_ar(model, prompt, W, N, G, rounds, **kw):
    s = la.Session(model, prompt, W=W, N=N, G=G, max_new=256, **kw)
    toks = list(s.la_get_state()["output"])
    for r in range(rounds):
        toks += s.la_step()
    st = s.la_stats()
    ar = la.Session(model, prompt, W=W, N=N, G=G, max_new=256, ar_only=True, **kw)
    ref = list(ar.la_get_state()["output"])
    while len(ref) < len(toks):
        ref += ar.la_step()
    _say(f"  {st['rounds']} rounds, {st['tokens']} tokens, {st['candidates']} candidates, {st['accepted']} accepted")
    return toks, ref[: len(toks)]


@pytest.fixture(scope="module")
def m34():
    dims = synthetic.PRESETS["codellama34b"]
    _say("loading the 34B-shaped model")
    m = la.DeviceModel(dims, seed=0)
    yield dims, m
    del m
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_34b_lookahead_equals_ar(m34):
    dims, m = m34
    prompt, copied = synthetic.copyspan_prompt(dims.vocab, 2048, 0)
    _say(f"34B GQA, 2048-token prompt ({copied * 100:.0f}% copied), W=15 N=7 G=15")
    toks, ref = _lookahead_vs_ar(m, prompt, 15, 7, 15, 20)
    assert toks == ref


@pytest.mark.timeout(900)
def test_34b_pool_from_prompt_equals_ar(m34):
    """The copy-span prompt's n-grams seeded into the pool: candidates every
    round, still the autoregressive tokens."""
    dims, m = m34
    prompt, _ = synthetic.copyspan_prompt(dims.vocab, 2048, 0)
    toks, ref = _lookahead_vs_ar(m, prompt, 15, 7, 15, 16, pool_from_prompt=True)
    assert toks == ref
