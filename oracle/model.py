"""Target model: a Llama-style decoder-only causal LM, computed plainly in fp64.

The pages treat the target as an unchanged causal model ("M7.3 - Lookahead
Decoding", 0x00 and 0x04C: one causal forward over the uncached rows with
past K/V, LM head over the rows, logits promoted to float32).  They do not
print its internals, so the architecture is the plain Llama reading: RMSNorm
(eps 1e-5), rotate-half RoPE (theta 10000) at each row's *logical* position,
grouped-query attention scaled by 1/sqrt(head_dim), SwiGLU MLP, untied LM
head, no biases.

Storage points (each stored value is rounded to the model dtype, "f32" or
"bf16"; everything between them is fp64):

    x    = E[token]
    per layer:
      n    = s(x * rs(x) * w_attn)                rs(x) = 1/sqrt(mean(x^2) + eps)
      q,k,v= s(n Wq^T), s(n Wk^T), s(n Wv^T)
      q,k  = s(rope(q, pos)), s(rope(k, pos))     K/V cache holds k and v
      o    = s(softmax(q K^T / sqrt(dh)) V)       over the row's visible keys
      h    = s(x + o Wo^T)
      n2   = s(h * rs(h) * w_mlp)
      a    = s(silu(n2 Wg^T) * (n2 Wu^T))
      x    = s(h + a Wd^T)
    logits = f32(s(x * rs(x) * w_final) Wlm^T)

The pages print no activations; the tests pin this forward against a second,
independent fp64 forward in torch (same storage points, its own matmuls,
rotation and attention), by textbook identities and by separate-forwards ==
dense-mask == AR.
"""
from __future__ import annotations

import numpy as np

from synthetic import ModelDims, f32_from_bf16_bits
from .numerics import round_to


def silu(g):
    return g / (1.0 + np.exp(-g))


def linear(x, w, dtype):
    """Stored projection: s(x W^T)."""
    return round_to(x @ w.T, dtype)


def linear_residual(x, w, r, dtype):
    """Residual update: s(r + x W^T)."""
    return round_to(r + x @ w.T, dtype)


def linear_swiglu(x, wg, wu, dtype):
    """SwiGLU activation: s(silu(x Wg^T) * (x Wu^T))."""
    return round_to(silu(x @ wg.T) * (x @ wu.T), dtype)


def logits_f32(x, w):
    """LM head, promoted to float32."""
    return (x @ w.T).astype(np.float32).astype(np.float64)


class KVCache:
    """Committed K/V per layer: k[l] and v[l] are [H_kv, T, dh] fp64 arrays (storage-rounded)."""

    def __init__(self, dims: ModelDims):
        self.k = [np.zeros((dims.n_kv_heads, 0, dims.head_dim)) for _ in range(dims.n_layers)]
        self.v = [np.zeros((dims.n_kv_heads, 0, dims.head_dim)) for _ in range(dims.n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[1]

    def append(self, layer: int, k_rows: np.ndarray, v_rows: np.ndarray):
        """k_rows, v_rows: [n, H_kv, dh] in logical order."""
        self.k[layer] = np.concatenate([self.k[layer], k_rows.transpose(1, 0, 2)], axis=1)
        self.v[layer] = np.concatenate([self.v[layer], v_rows.transpose(1, 0, 2)], axis=1)

    def copy(self) -> "KVCache":
        c = KVCache.__new__(KVCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c


class OracleModel:
    """fp64 forward with storage rounding.  `weights` comes from synthetic.model_weights."""

    def __init__(self, dims: ModelDims, weights: dict, cache_limit_bytes: float = 12e9):
        self.dims = dims
        self.w = weights
        self._cache = {}
        n_params = (2 * dims.vocab * dims.d_model + dims.n_layers * (
            2 * dims.q_dim * dims.d_model + 2 * dims.kv_dim * dims.d_model + 3 * dims.d_ff * dims.d_model))
        self._cache_all = n_params * 8 <= cache_limit_bytes

    # weights as fp64 ----------------------------------------------------
    def _f64(self, a):
        if a.dtype == np.uint16:
            return f32_from_bf16_bits(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)

    def weight(self, name: str, layer: int | None = None) -> np.ndarray:
        key = (name, layer)
        if key in self._cache:
            return self._cache[key]
        src = self.w[name] if layer is None else self.w["layers"][layer][name]
        a = self._f64(src)
        if self._cache_all:
            self._cache[key] = a
        return a

    # building blocks ----------------------------------------------------
    def s(self, x):
        return round_to(x, self.dims.dtype)

    def rms_norm(self, x, w):
        rs = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + self.dims.eps)
        return self.s(x * rs * w)

    def rope(self, x, positions):
        """Rotate-half RoPE.  x: [n, heads, dh]; positions: [n] logical positions."""
        dh = x.shape[-1]
        half = dh // 2
        inv_freq = self.dims.rope_theta ** (-np.arange(half, dtype=np.float64) * 2.0 / dh)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
        cos = np.cos(ang)[:, None, :]
        sin = np.sin(ang)[:, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


    # one forward over new rows --------------------------------------------
    def forward(self, tokens, positions, cache: KVCache | None, visible: np.ndarray,
                logit_rows=None):
        """Forward `tokens` (new, uncached rows) against committed K/V in `cache`.

        Every new row sees every committed key; among the new rows, row i sees
        row j iff visible[i, j].  Returns (logits [n_logit, V] float32-valued
        fp64, new_k, new_v) where new_k[l], new_v[l] are [n, H_kv, dh] for each
        layer (the rows' own K/V, not yet committed).
        """
        d = self.dims
        tokens = np.asarray(tokens, dtype=np.int64)
        n = len(tokens)
        positions = np.asarray(positions, dtype=np.int64)
        visible = np.asarray(visible, dtype=bool)
        assert visible.shape == (n, n)
        group = d.n_heads // d.n_kv_heads
        scale = 1.0 / np.sqrt(d.head_dim)
        x = self.s(self.weight("embed")[tokens])
        new_k, new_v = [], []
        for l in range(d.n_layers):
            nrm = self.rms_norm(x, self.weight("attn_norm", l))
            q = linear(nrm, self.weight("wq", l), d.dtype).reshape(n, d.n_heads, d.head_dim)
            k = linear(nrm, self.weight("wk", l), d.dtype).reshape(n, d.n_kv_heads, d.head_dim)
            v = linear(nrm, self.weight("wv", l), d.dtype).reshape(n, d.n_kv_heads, d.head_dim)
            q = self.s(self.rope(q, positions))
            k = self.s(self.rope(k, positions))
            new_k.append(k)
            new_v.append(v)
            if cache is not None and cache.length > 0:
                kc, vc = cache.k[l], cache.v[l]          # [Hkv, T, dh]
            else:
                kc = np.zeros((d.n_kv_heads, 0, d.head_dim))
                vc = np.zeros((d.n_kv_heads, 0, d.head_dim))
            T = kc.shape[1]
            o = np.zeros((n, d.n_heads, d.head_dim))
            for h in range(d.n_heads):
                g = h // group
                keys = np.concatenate([kc[g], k[:, g, :]], axis=0)      # [T+n, dh]
                vals = np.concatenate([vc[g], v[:, g, :]], axis=0)
                sc = (q[:, h, :] @ keys.T) * scale                      # [n, T+n]
                allowed = np.concatenate([np.ones((n, T), bool), visible], axis=1)
                sc = np.where(allowed, sc, -np.inf)
                m = sc.max(axis=1, keepdims=True)
                p = np.exp(sc - m)
                p = p / p.sum(axis=1, keepdims=True)
                o[:, h, :] = p @ vals
            o = self.s(o).reshape(n, d.q_dim)
            h_res = linear_residual(o, self.weight("wo", l), x, d.dtype)
            n2 = self.rms_norm(h_res, self.weight("mlp_norm", l))
            a = linear_swiglu(n2, self.weight("w_gate", l), self.weight("w_up", l), d.dtype)
            x = linear_residual(a, self.weight("w_down", l), h_res, d.dtype)
        rows = np.arange(n) if logit_rows is None else np.asarray(logit_rows, dtype=np.int64)
        xf = self.rms_norm(x[rows], self.weight("final_norm"))
        logits = logits_f32(xf, self.weight("lm_head"))
        return logits, new_k, new_v

    # conveniences ---------------------------------------------------------
    def prefill(self, tokens):
        """Plain causal forward over a prompt.  Returns (cache, logits of every row)."""
        n = len(tokens)
        cache = KVCache(self.dims)
        logits, nk, nv = self.forward(tokens, np.arange(n), None, np.tril(np.ones((n, n), bool)))
        for l in range(self.dims.n_layers):
            cache.append(l, nk[l], nv[l])
        return cache, logits

    def sequence_logits(self, tokens):
        """Separate-forward reference: logits of the last row of a plain causal forward."""
        n = len(tokens)
        logits, _, _ = self.forward(tokens, np.arange(n), None, np.tril(np.ones((n, n), bool)),
                                    logit_rows=[n - 1])
        return logits[0]
