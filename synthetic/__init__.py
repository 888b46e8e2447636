"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only *generates inputs*: model weights, prompts, attention-op
tensors, logits and candidate sets for unit cases.  It holds none of the
lookahead method's arithmetic (no forward pass, no verification, no pool or
window logic), so both sides may import it without sharing method code.

Every array is a pure function of (seed, what it is).  Each tensor draws from
its own PCG64 stream whose SeedSequence spawn key names the tensor, so a
single layer can be regenerated without materialising the others.

Workloads (the pages evaluate on MT-Bench / code-completion suites with
trained LLaMA weights, neither of which is available here; these seeded
sources stand in for them):

* random-init Llama-style decoders, weights N(0, 0.02), norm weights 1;
* prompts from an order-2 Markov chain over the vocabulary in which every
  state (a, b) has 4 distinct successors with Dirichlet(0.5) weights, so
  n-grams recur the way they do in natural text;
* for the 34B-shaped workload, the same chain plus copied spans of length
  8..32 from earlier in the prompt (about 30% of tokens), mimicking the
  repetitive structure of code.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "ModelDims", "PRESETS", "tensor_rng", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "weight_tensor", "model_weights", "markov_prompt", "copyspan_prompt",
    "attention_op_inputs", "LAYER_TENSORS", "GLOBAL_TENSORS",
]

# --------------------------------------------------------------------------
# model shapes
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ModelDims:
    """Shape of a Llama-style decoder-only causal LM (RMSNorm, RoPE, SwiGLU)."""
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    dtype: str            # storage dtype: "f32" or "bf16"
    eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


PRESETS = {
    # 2 layers, d 64, 4 heads x 16, MLP 256, vocab 256, fp32 weights
    "tiny": ModelDims(2, 64, 4, 4, 16, 256, 256, "f32"),
    # Llama-2-7B shape, bf16
    "llama7b": ModelDims(32, 4096, 32, 32, 128, 11008, 32000, "bf16"),
    # CodeLlama-34B shape (GQA, 8 KV heads), bf16
    "codellama34b": ModelDims(48, 8192, 64, 8, 128, 22016, 32000, "bf16"),
    # 7B widths at 2 layers: the oracle can run it end to end in seconds
    "llama7b_2l": ModelDims(2, 4096, 32, 32, 128, 11008, 32000, "bf16"),
    # a small bf16 model that still spans several GEMM / attention tiles
    "small_bf16": ModelDims(2, 256, 4, 2, 64, 512, 1024, "bf16"),
}

# tensor kinds (the spawn key of each tensor's stream is (kind, layer))
GLOBAL_TENSORS = {"embed": 0, "lm_head": 1, "final_norm": 2}
LAYER_TENSORS = {"attn_norm": 3, "wq": 4, "wk": 5, "wv": 6, "wo": 7,
                 "mlp_norm": 8, "w_gate": 9, "w_up": 10, "w_down": 11}

_STREAM_WEIGHTS = 1
_STREAM_CHAIN = 2
_STREAM_PROMPT = 3
_STREAM_ATTN = 4
_STREAM_MISC = 5


def tensor_rng(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, key...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed), spawn_key=tuple(int(k) for k in key))))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1).astype(np.uint32) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _shape_of(dims: ModelDims, name: str):
    d = dims.d_model
    return {
        "embed": (dims.vocab, d), "lm_head": (dims.vocab, d), "final_norm": (d,),
        "attn_norm": (d,), "mlp_norm": (d,),
        "wq": (dims.q_dim, d), "wk": (dims.kv_dim, d), "wv": (dims.kv_dim, d),
        "wo": (d, dims.q_dim),
        "w_gate": (dims.d_ff, d), "w_up": (dims.d_ff, d), "w_down": (d, dims.d_ff),
    }[name]


def weight_tensor(dims: ModelDims, name: str, layer: int = 0, seed: int = 0) -> np.ndarray:
    """One weight tensor, nn.Linear layout [out_features, in_features].

    Matrices and the embedding are N(0, 0.02) drawn in float32; norm weights
    are 1.  For bf16 models the result is uint16 bf16 bit patterns, otherwise
    float32.
    """
    shape = _shape_of(dims, name)
    if name in ("final_norm", "attn_norm", "mlp_norm"):
        w = np.ones(shape, np.float32)
    else:
        kind = GLOBAL_TENSORS.get(name, LAYER_TENSORS.get(name))
        rng = tensor_rng(seed, _STREAM_WEIGHTS, kind, layer)
        w = np.empty(shape, np.float32)
        rng.standard_normal(out=w, dtype=np.float32)
        w *= np.float32(0.02)
    if dims.dtype == "bf16":
        return bf16_bits_from_f32(w)
    return w


def model_weights(dims: ModelDims, seed: int = 0, threads: int | None = None, layers=None) -> dict:
    """All weights: {"embed", "lm_head", "final_norm", "layers": [ {name: array} ]}.

    Generation is spread over threads (numpy releases the GIL while drawing).
    `layers` restricts which layers are produced (others are None).
    """
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    layer_ids = range(dims.n_layers) if layers is None else list(layers)
    jobs = [(n, 0) for n in GLOBAL_TENSORS] + [(n, l) for l in layer_ids for n in LAYER_TENSORS]
    with ThreadPoolExecutor(max(1, threads)) as ex:
        outs = list(ex.map(lambda j: weight_tensor(dims, j[0], j[1], seed), jobs))
    res = {"layers": [None] * dims.n_layers}
    for (n, l), a in zip(jobs, outs):
        if n in GLOBAL_TENSORS:
            res[n] = a
        else:
            if res["layers"][l] is None:
                res["layers"][l] = {}
            res["layers"][l][n] = a
    return res


# --------------------------------------------------------------------------
# prompts
# --------------------------------------------------------------------------


def _markov_state(vocab: int, a: int, b: int, chain_seed: int):
    """Successors (4 distinct ids) and their Dirichlet(0.5) weights for state (a, b)."""
    rng = tensor_rng(chain_seed, _STREAM_CHAIN, a, b)
    succ = rng.choice(vocab, size=4, replace=False)
    w = rng.gamma(0.5, size=4)
    w = w / w.sum()
    return succ, w


def _markov_next(vocab, a, b, u, chain_seed):
    succ, w = _markov_state(vocab, a, b, chain_seed)
    c = np.cumsum(w)
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    return int(succ[min(i, 3)])


def markov_prompt(vocab: int, length: int, seed: int = 0, chain_seed: int = 0) -> list:
    """Prompt from the seeded order-2 Markov chain; the first two tokens are uniform."""
    rng = tensor_rng(seed, _STREAM_PROMPT, 0)
    toks = [int(rng.integers(vocab)), int(rng.integers(vocab))][:length]
    while len(toks) < length:
        toks.append(_markov_next(vocab, toks[-2], toks[-1], rng.random(), chain_seed))
    return toks


def copyspan_prompt(vocab: int, length: int, seed: int = 0, chain_seed: int = 0):
    """Markov chain plus copied spans (length U{8..32}) from earlier in the prompt.

    Once the prompt holds 64 tokens, each step copies a span with probability
    0.3/14.3 (so about 30% of tokens are copies, a span averaging 20 tokens),
    otherwise emits one Markov token conditioned on the last two tokens.
    Returns (tokens, realized copied fraction).
    """
    rng = tensor_rng(seed, _STREAM_PROMPT, 1)
    p_copy = 0.3 / 14.3
    toks = [int(rng.integers(vocab)), int(rng.integers(vocab))][:length]
    copied = 0
    while len(toks) < length:
        if len(toks) >= 64 and rng.random() < p_copy:
            L = int(rng.integers(8, 33))
            start = int(rng.integers(0, len(toks) - L + 1))
            span = toks[start:start + L][: length - len(toks)]
            toks.extend(span)
            copied += len(span)
        else:
            toks.append(_markov_next(vocab, toks[-2], toks[-1], rng.random(), chain_seed))
    return toks, copied / max(1, length)


# --------------------------------------------------------------------------
# isolated attention-op inputs
# --------------------------------------------------------------------------


def attention_op_inputs(n_rows: int, n_heads: int, n_kv_heads: int, head_dim: int,
                        prefix_len: int, seed: int = 0, dtype: str = "bf16"):
    """Q [n_rows][H][dh], prefix K/V [Hkv][prefix_len][dh], new-row K/V [n_rows][Hkv][dh].

    All N(0, 1); bf16 bit patterns (uint16) or float32.  Row i of the new K/V
    belongs to query row i (rows are in the order the caller defines).
    """
    def draw(k, shape):
        a = np.empty(shape, np.float32)
        tensor_rng(seed, _STREAM_ATTN, k).standard_normal(out=a, dtype=np.float32)
        return bf16_bits_from_f32(a) if dtype == "bf16" else a
    q = draw(0, (n_rows, n_heads, head_dim))
    kp = draw(1, (n_kv_heads, prefix_len, head_dim))
    vp = draw(2, (n_kv_heads, prefix_len, head_dim))
    kn = draw(3, (n_rows, n_kv_heads, head_dim))
    vn = draw(4, (n_rows, n_kv_heads, head_dim))
    return q, kp, vp, kn, vn


def misc_rng(seed: int, *key: int) -> np.random.Generator:
    """Stream for ad-hoc unit-test inputs (window tokens, candidate sets, logits)."""
    return tensor_rng(seed, _STREAM_MISC, *key)
