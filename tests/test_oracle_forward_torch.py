"""The oracle's model forward against a second, independent forward in torch (CPU, fp64).

The pages print no activations, so the oracle's Llama forward
(oracle/model.py) is pinned here by a separate implementation that imports
nothing from oracle/: torch fp64 tensors, torch's own matmul, RMSNorm via
rsqrt, rotate-half RoPE written from the rotation definition, grouped-query
attention through torch.nn.functional.scaled_dot_product_attention with a
boolean visibility mask, SwiGLU, an untied LM head.  Values are rounded to the
model's storage dtype at the same storage points the model's description
lists (embedding, normed rows, q/k/v, rotated q/k, attention output, the
residual stream, the SwiGLU activation) and logits are promoted to float32.

The packed round is built here too, straight from the visibility sets and
logical positions of "M7.3 - Lookahead Decoding" 0x04A (Vis(b_j),
Vis(u_(r,j)), Vis(v_(c,s)); pos(b_j) = p + j, pos(u_(r,j)) = p + j + r,
pos(v_(c,s)) = p + 1 + s), and the reference runs the committed prompt and
the round's rows as ONE torch forward (prompt causal, every round row seeing
the whole prompt), whereas the oracle prefills the prompt and then forwards
the round against its cache.

Agreement: the committed K/V rows, the round's new K/V rows and the logits.
Two fp64 evaluations with different summation orders agree to ~1e-15
relative before rounding, so every stored value has the same bits except
with probability ~1e-13 per value; the float32 logits are allowed one fp32
ulp (a pre-rounding value that sits on a rounding boundary), and nearly all
of them must be bit-identical.  A dropped term, a wrong sign in the rotation,
a swapped gate/up, a wrong attention scale or GQA head map, or a mask edge
too many or too few moves the logits by orders of magnitude more.
"""
import math

import numpy as np
import pytest

import synthetic

torch = pytest.importorskip("torch")

from oracle.model import OracleModel  # noqa: E402  (the implementation under test)


# ---------------------------------------------------------------- storage rounding

def _round_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """float64 -> nearest bfloat16 value (ties to even), one rounding, on the
    float64 bit pattern: keep the sign, the exponent and the top 7 of the 52
    mantissa bits, rounding at bit 45.  (torch's own float64 -> bfloat16
    conversion goes through float32 first, i.e. rounds twice.)"""
    u = x.contiguous().view(torch.int64)
    lsb = (u >> 45) & 1
    u = (u + ((1 << 44) - 1) + lsb) & ~((1 << 45) - 1)
    return u.view(torch.float64)


def _storage(dtype):
    if dtype == "bf16":
        return _round_bf16_bits
    return lambda t: t.to(torch.float32).to(torch.float64)


def test_bf16_rounding_helper():
    """The helper agrees with torch's float32 -> bfloat16 conversion (a single
    rounding there) on float32-representable inputs, ties included."""
    g = torch.Generator().manual_seed(0)
    x32 = torch.cat([torch.randn(100000, generator=g), torch.randn(1000, generator=g) * 1e-20,
                     torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0])]).to(torch.float32)
    want = x32.to(torch.bfloat16).to(torch.float64)
    got = _round_bf16_bits(x32.to(torch.float64))
    assert torch.equal(got, want)


# ---------------------------------------------------------------- reference forward

class TorchLlama:
    """fp64 Llama-style decoder over one token sequence with an explicit
    boolean visibility mask (mask[i, j]: row i attends row j)."""

    def __init__(self, dims, weights):
        self.d = dims
        self.s = _storage(dims.dtype)

        def t(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64)
            return torch.from_numpy(a).to(torch.float64)
        self.embed = t(weights["embed"])
        self.lm_head = t(weights["lm_head"])
        self.final_norm = t(weights["final_norm"])
        self.layers = [{k: t(v) for k, v in lw.items()} for lw in weights["layers"]]

    def norm(self, x, w):
        return self.s(x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + self.d.eps) * w)

    def rotate(self, x, pos):
        """x [n, heads, dh] -> x cos + rotate_half(x) sin, angle pos * theta^(-2i/dh)."""
        dh = x.shape[-1]
        i = torch.arange(dh // 2, dtype=torch.float64)
        inv = torch.exp(-(2.0 * i / dh) * math.log(self.d.rope_theta))
        ang = pos.to(torch.float64)[:, None] * inv[None, :]
        cos = torch.cat([ang.cos(), ang.cos()], dim=-1)[:, None, :]
        sin = torch.cat([ang.sin(), ang.sin()], dim=-1)[:, None, :]
        half = torch.cat([-x[..., dh // 2:], x[..., : dh // 2]], dim=-1)
        return x * cos + half * sin

    def __call__(self, tokens, pos, mask, out_rows):
        d = self.d
        n = len(tokens)
        tok = torch.as_tensor(tokens, dtype=torch.long)
        pos = torch.as_tensor(pos, dtype=torch.long)
        mask = torch.as_tensor(mask, dtype=torch.bool)
        group = d.n_heads // d.n_kv_heads
        x = self.s(self.embed[tok])
        ks, vs = [], []
        for lw in self.layers:
            h = self.norm(x, lw["attn_norm"])
            q = self.s(h @ lw["wq"].T).view(n, d.n_heads, d.head_dim)
            k = self.s(h @ lw["wk"].T).view(n, d.n_kv_heads, d.head_dim)
            v = self.s(h @ lw["wv"].T).view(n, d.n_kv_heads, d.head_dim)
            q = self.s(self.rotate(q, pos))
            k = self.s(self.rotate(k, pos))
            ks.append(k)
            vs.append(v)
            # [1, heads, n, dh]; each query head reads KV head h // group
            qh = q.permute(1, 0, 2)[None]
            kh = k.permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
            vh = v.permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
            o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask[None, None],
                                                                 scale=1.0 / math.sqrt(d.head_dim))
            o = self.s(o[0].permute(1, 0, 2).reshape(n, d.n_heads * d.head_dim))
            x = self.s(x + o @ lw["wo"].T)
            h2 = self.norm(x, lw["mlp_norm"])
            g = h2 @ lw["w_gate"].T
            a = self.s(g * torch.sigmoid(g) * (h2 @ lw["w_up"].T))
            x = self.s(x + a @ lw["w_down"].T)
        xf = self.norm(x[torch.as_tensor(out_rows, dtype=torch.long)], self.final_norm)
        logits = (xf @ self.lm_head.T).to(torch.float32).to(torch.float64)
        return logits.numpy(), [k.numpy() for k in ks], [v.numpy() for v in vs]


# ---------------------------------------------------------------- packed round from the page's sets

def packed_round(p, x_t, levels, starts, cands):
    """Rows of one round in the page's dense order (ordinary row, level-major
    lookahead rows, candidate-major verification rows) with tokens, logical
    positions and the Vis sets among the round's rows.  levels[0] holds
    b_1..; levels[r] (r >= 1) holds u_(r, starts[r] + i)."""
    rows = [("b", 0, 0, x_t)]                          # (kind, level or candidate, column or offset, token)
    for j, t in enumerate(levels[0]):
        rows.append(("b", 0, j + 1, t))
    for r in range(1, len(levels)):
        for i, t in enumerate(levels[r] or []):
            rows.append(("u", r, starts[r] + i, t))
    for c, suf in enumerate(cands):
        for s, t in enumerate(suf):
            rows.append(("v", c, s, t))
    pos = []
    for kind, a, b, _ in rows:
        pos.append(p + b if kind == "b" else p + b + a if kind == "u" else p + 1 + b)

    def sees(i, j):
        ki, ai, bi, _ = rows[i]
        kj, aj, bj, _ = rows[j]
        if ki == "b":
            return kj == "b" and bj <= bi
        if ki == "u":
            return (kj == "b" and bj <= bi) or (kj == "u" and bj == bi and aj <= ai)
        return (kj == "b" and bj == 0) or (kj == "v" and aj == ai and bj <= bi)
    Q = len(rows)
    vis = np.array([[sees(i, j) for j in range(Q)] for i in range(Q)], bool)
    return [r[3] for r in rows], pos, vis


def _compare(om, tm, prompt, tokens, pos, vis, out_rows):
    P, Q = len(prompt), len(tokens)
    cache, _ = om.prefill(prompt)
    lg_o, nk_o, nv_o = om.forward(tokens, pos, cache, vis, logit_rows=out_rows)
    # one causal + packed forward over prompt and round in the reference
    mask = np.zeros((P + Q, P + Q), bool)
    mask[:P, :P] = np.tril(np.ones((P, P), bool))
    mask[P:, :P] = True
    mask[P:, P:] = vis
    lg_t, k_t, v_t = tm(list(prompt) + list(tokens), list(range(P)) + list(pos), mask, [P + i for i in out_rows])
    for l in range(om.dims.n_layers):
        assert np.array_equal(cache.k[l], k_t[l][:P].transpose(1, 0, 2)), l     # committed K/V
        assert np.array_equal(cache.v[l], v_t[l][:P].transpose(1, 0, 2)), l
        assert np.array_equal(nk_o[l], k_t[l][P:]), l                            # the round's K/V
        assert np.array_equal(nv_o[l], v_t[l][P:]), l
    d = np.abs(lg_o - lg_t)
    ulp = np.abs(lg_t) * 2.0 ** -23 + 1e-30
    assert np.all(d <= ulp), float(d.max())
    assert np.mean(d > 0) < 1e-4
    return float(d.max())


def _models(name):
    dims = synthetic.PRESETS[name]
    w = synthetic.model_weights(dims, 0)
    return OracleModel(dims, w), TorchLlama(dims, w)


@pytest.fixture(scope="module")
def tiny():
    return _models("tiny")


@pytest.fixture(scope="module")
def small_bf16():
    return _models("small_bf16")


def test_vis_sets_of_the_page_example():
    """The W=5, N=4, G=2 steady layout of 0x04A: 21 rows; b_2 sees b_0..b_2;
    u_(2,3) sees b_0..b_3, u_(1,3), u_(2,3); v_(1,2) sees b_0 and v_(1,0..2)."""
    tok, pos, vis = packed_round(10, 1, [[2, 3, 4, 5], [6, 7, 8, 9, 10], [11, 12, 13, 14, 15]], [1, 0, 0],
                                 [(20, 21, 22), (23, 24, 25)])
    assert len(tok) == 21
    b = lambda j: j                        # noqa: E731
    u = lambda r, j: 5 + 5 * (r - 1) + j   # noqa: E731
    v = lambda c, s: 15 + 3 * c + s        # noqa: E731
    assert set(np.flatnonzero(vis[b(2)])) == {b(0), b(1), b(2)}
    assert set(np.flatnonzero(vis[u(2, 3)])) == {b(0), b(1), b(2), b(3), u(1, 3), u(2, 3)}
    assert set(np.flatnonzero(vis[v(1, 2)])) == {b(0), v(1, 0), v(1, 1), v(1, 2)}
    assert pos[u(2, 3)] == 10 + 3 + 2 and pos[v(1, 2)] == 10 + 3 and pos[b(4)] == 14


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_fp32_round(tiny, seed):
    om, tm = tiny
    rng = synthetic.misc_rng(seed, 90)
    prompt = synthetic.markov_prompt(256, 24, seed)
    W, N, G = 5, 4, 3
    lv = [[int(t) for t in rng.integers(0, 256, W - 1)]] + [[int(t) for t in rng.integers(0, 256, W)]
                                                            for _ in range(N - 2)]
    cands = [tuple(int(t) for t in rng.integers(0, 256, N - 1)) for _ in range(G)]
    tok, pos, vis = packed_round(len(prompt), int(rng.integers(256)), lv, [1] + [0] * (N - 2), cands)
    err = _compare(om, tm, prompt, tok, pos, vis, list(range(len(tok))))
    print(f"tiny fp32: max |oracle - torch| = {err:.3g}")


def test_small_bf16_gqa_round(small_bf16):
    """bf16 storage, 4 query heads on 2 KV heads, head dim 64; a warmup-stage
    layout (levels [6, 7, -]) and a steady one with candidates."""
    om, tm = small_bf16
    rng = synthetic.misc_rng(2, 91)
    prompt = synthetic.markov_prompt(1024, 40, 3)
    for levels, starts, C in [([7, 6, 0], [1, 0, 0], 0), ([5, 6, 6], [1, 0, 0], 4)]:
        lv = [[int(t) for t in rng.integers(0, 1024, n)] if n else None for n in levels]
        cands = [tuple(int(t) for t in rng.integers(0, 1024, 3)) for _ in range(C)]
        tok, pos, vis = packed_round(len(prompt), int(rng.integers(1024)), lv, starts, cands)
        err = _compare(om, tm, prompt, tok, pos, vis, list(range(len(tok))))
        print(f"small bf16 {levels}: max |oracle - torch| = {err:.3g}")


@pytest.mark.slow
def test_llama7b_width_2layer_round():
    """7B widths (d 4096, 32 heads x 128, MLP 11008, vocab 32000), 2 layers,
    bf16: the W=7, N=5, G=7 steady round (56 rows) after a 48-token prompt;
    logits of the out, inp and guess rows."""
    om, tm = _models("llama7b_2l")
    rng = synthetic.misc_rng(3, 92)
    prompt = synthetic.markov_prompt(32000, 48, 0)
    W, N, G = 7, 5, 7
    lv = [[int(t) for t in rng.integers(0, 32000, W - 1)]] + [[int(t) for t in rng.integers(0, 32000, W)]
                                                              for _ in range(N - 2)]
    cands = [tuple(int(t) for t in rng.integers(0, 32000, N - 1)) for _ in range(G)]
    tok, pos, vis = packed_round(len(prompt), int(rng.integers(32000)), lv, [1] + [0] * (N - 2), cands)
    Q = len(tok)
    assert Q == 56
    deepest = list(range(1 + (W - 1) + (N - 3) * W, 1 + (W - 1) + (N - 2) * W))
    out_rows = [0] + deepest + list(range(Q - G * (N - 1), Q))
    err = _compare(om, tm, prompt, tok, pos, vis, out_rows)
    print(f"7B-width 2-layer bf16: max |oracle - torch| = {err:.3g}")
