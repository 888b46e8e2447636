"""Thin ctypes binding of the C ABI in include/la.h (argument marshalling only).

Every step of the lookahead path runs in the HIP library; this module only
allocates device buffers through torch, passes raw pointers and copies
small host arrays.  The library must be built (exact_lookahead_decoding_amd
.build); importing without it raises.
"""
from __future__ import annotations

import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

from . import build as _build

LA_OK, LA_EINVAL, LA_ESTATE, LA_EPLAN, LA_EOVERFLOW, LA_EDEVICE = 0, -1, -2, -3, -4, -5
LA_MAX_N = 16
LA_MAX_EMIT = 32
LA_NOALLOC_SCRATCH_BYTES = 32 << 20
LA_DTYPE_F32, LA_DTYPE_BF16 = 0, 1
LA_VERIFY_GREEDY, LA_VERIFY_SAMPLE = 0, 1

_ERRNAMES = {LA_EINVAL: "LA_EINVAL", LA_ESTATE: "LA_ESTATE", LA_EPLAN: "LA_EPLAN",
             LA_EOVERFLOW: "LA_EOVERFLOW", LA_EDEVICE: "LA_EDEVICE"}


class LaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


class la_model_dims(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("d_ff", C.c_int32), ("vocab", C.c_int32), ("dtype", C.c_int32),
                ("eps", C.c_float), ("rope_theta", C.c_float)]


class la_model(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("embed", "lm_head", "final_norm", "attn_norm", "wqkv", "wo", "mlp_norm",
                                          "w_gate_up", "w_down", "packed")]


class la_config(C.Structure):
    _fields_ = [("W", C.c_int32), ("N", C.c_int32), ("G", C.c_int32), ("max_new", C.c_int32),
                ("verify_mode", C.c_int32), ("ar_only", C.c_int32), ("temperature", C.c_double),
                ("seed", C.c_uint64), ("max_prompt", C.c_int32), ("pool_from_prompt", C.c_int32),
                ("advance_by_accepted", C.c_int32), ("cap_full_match", C.c_int32), ("pool_from_output", C.c_int32)]


class la_sizes(C.Structure):
    _fields_ = [("kv_bytes", C.c_uint64), ("arena_bytes", C.c_uint64), ("t_cap", C.c_int32), ("q_max", C.c_int32),
                ("n_logit_max", C.c_int32), ("reserved", C.c_int32)]


class la_accept(C.Structure):
    _fields_ = [("round_id", C.c_int32), ("h", C.c_int32), ("winner", C.c_int32), ("n_emit", C.c_int32),
                ("emitted", C.c_int32 * LA_MAX_EMIT)]


class la_round_info(C.Structure):
    _fields_ = [("round_id", C.c_int32), ("p", C.c_int32), ("Q", C.c_int32), ("C", C.c_int32),
                ("n_inp", C.c_int32), ("n_logit", C.c_int32), ("warm", C.c_int32), ("reserved", C.c_int32),
                ("logits", C.c_void_p)]


class la_stats_t(C.Structure):
    _fields_ = [("rounds", C.c_int64), ("tokens", C.c_int64), ("candidates", C.c_int64), ("accepted", C.c_int64),
                ("hist", C.c_int32 * LA_MAX_EMIT), ("paused", C.c_int64)]


class la_batch_round(C.Structure):
    _fields_ = [("Q", C.c_int32), ("found", C.c_int32), ("verified", C.c_int32), ("paused", C.c_int32),
                ("h", C.c_int32), ("reserved", C.c_int32 * 3)]


class la_state_t(C.Structure):
    _fields_ = [("round_id", C.c_int32), ("kv_len", C.c_int32), ("n_out", C.c_int32), ("R", C.c_int32),
                ("level_sizes", C.c_int32 * LA_MAX_N), ("warm", C.c_int32), ("win_stride", C.c_int32)]


class la_profile_t(C.Structure):
    _fields_ = [("gemm_ms", C.c_double), ("gemm_bytes", C.c_double), ("gemm_flops", C.c_double),
                ("attn_ms", C.c_double), ("attn_bytes", C.c_double), ("attn_flops", C.c_double),
                ("gemm_launches", C.c_int64), ("attn_launches", C.c_int64)]


class la_rows_desc(C.Structure):
    _fields_ = [("p", C.c_int32), ("R", C.c_int32), ("sizes", C.c_int32 * LA_MAX_N),
                ("starts", C.c_int32 * LA_MAX_N), ("C", C.c_int32), ("S", C.c_int32), ("x_t", C.c_int32),
                ("win_stride", C.c_int32)]


class la_rows_info(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "Q", "NB", "maxp", "n_logit", "n_inp", "n_cols", "mask_words", "total_words",
        "off_tok", "off_pos", "off_role", "off_level", "off_col", "off_cand", "off_off", "off_branch",
        "off_path", "off_path_len", "off_logit_rows", "off_mask", "off_tile_meta", "off_tile_path")]


EXPORTS = ["la_query_sizes", "la_init", "la_destroy", "la_step", "la_generate", "la_predict", "la_verify",
           "la_commit", "la_pool_lookup", "la_pool_insert", "la_get_state", "la_stats", "la_last_error",
           "la_rows_query", "la_build_rows", "la_attention_workspace", "la_attention", "la_linear_workspace",
           "la_linear", "la_packed_linear_bytes", "la_pack_linear", "la_linear_packed", "la_packed_weight_bytes",
           "la_pack_weights", "la_profile", "la_profile_read", "la_attention_noalloc", "la_batch_bytes",
           "la_batch_init", "la_batch_destroy", "la_batch_plan", "la_batch_step"]
LA_LINEAR_STORE, LA_LINEAR_RESIDUAL, LA_LINEAR_SWIGLU, LA_LINEAR_F32 = 0, 1, 2, 3

_lib = None


def library_path() -> str:
    return _build.LIB


def load() -> C.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_lookahead_decoding_amd.build`")
    lib = C.CDLL(path)
    P, I32, VP = C.POINTER, C.c_int32, C.c_void_p
    sig = {
        "la_query_sizes": ([P(la_config), P(la_model_dims), P(la_sizes)], I32),
        "la_init": ([P(la_config), P(la_model_dims), P(la_model), VP, VP, P(I32), I32, VP, P(VP)], I32),
        "la_destroy": ([VP], None),
        "la_step": ([VP, P(I32), I32, P(I32)], I32),
        "la_generate": ([VP, P(I32), I32, P(I32)], I32),
        "la_predict": ([VP, P(la_round_info)], I32),
        "la_verify": ([VP, VP, I32, P(I32), I32, P(la_accept), P(I32)], I32),
        "la_commit": ([VP, P(la_accept)], I32),
        "la_pool_lookup": ([VP, I32, P(I32), P(I32)], I32),
        "la_pool_insert": ([VP, P(I32), P(I32), I32], I32),
        "la_get_state": ([VP, P(la_state_t), P(I32), P(I32), I32], I32),
        "la_stats": ([VP, P(la_stats_t)], I32),
        "la_last_error": ([VP], C.c_char_p),
        "la_rows_query": ([P(la_rows_desc), P(la_rows_info)], I32),
        "la_build_rows": ([P(la_rows_desc), VP, VP, VP, VP, P(la_rows_info)], I32),
        "la_attention_workspace": ([I32, I32, I32, I32, I32], C.c_size_t),
        "la_attention": ([I32, VP, VP, VP, I32, VP, VP, I32, I32, I32, I32, VP, P(la_rows_info), I32, VP, VP,
                          C.c_size_t, VP], I32),
        "la_attention_noalloc": ([I32, VP, VP, VP, I32, VP, VP, I32, I32, I32, I32, VP, P(la_rows_info), I32, VP,
                                  VP], I32),
        "la_linear_workspace": ([I32, I32, I32, I32, I32], C.c_size_t),
        "la_linear": ([I32, I32, VP, VP, VP, VP, I32, I32, I32, VP, C.c_size_t, VP], I32),
        "la_packed_linear_bytes": ([I32, I32, I32, I32], C.c_size_t),
        "la_pack_linear": ([I32, I32, VP, I32, I32, VP, VP], I32),
        "la_linear_packed": ([I32, I32, VP, VP, VP, VP, I32, I32, I32, VP, C.c_size_t, VP], I32),
        "la_packed_weight_bytes": ([P(la_model_dims)], C.c_uint64),
        "la_pack_weights": ([P(la_model_dims), P(la_model), VP, VP], I32),
        "la_profile": ([VP, I32], I32),
        "la_profile_read": ([VP, P(la_profile_t)], I32),
        "la_batch_bytes": ([P(la_model_dims), I32], C.c_uint64),
        "la_batch_init": ([P(la_model_dims), P(la_model), I32, VP, C.c_uint64, VP, P(VP)], I32),
        "la_batch_destroy": ([VP], None),
        "la_batch_plan": ([I32, I32, I32, P(I32), P(I32), P(I32), P(I32)], I32),
        "la_batch_step": ([VP, P(VP), I32, I32, P(I32), P(I32), P(la_batch_round)], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(rc, ctx=None):
    if rc != LA_OK:
        msg = load().la_last_error(ctx)
        raise LaError(rc, msg.decode() if msg else "")


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


# ----------------------------------------------------------------- model


def dims_struct(d) -> la_model_dims:
    return la_model_dims(d.n_layers, d.d_model, d.n_heads, d.n_kv_heads, d.head_dim, d.d_ff, d.vocab,
                         LA_DTYPE_BF16 if d.dtype == "bf16" else LA_DTYPE_F32, d.eps, d.rope_theta)


class DeviceModel:
    """Weights on the device in the layout of la_model (marshalling of synthetic weights)."""

    def __init__(self, dims, seed=0, device="cuda", threads=None, weights=None):
        import synthetic
        self.dims = dims
        bf = dims.dtype == "bf16"
        tdt = torch.bfloat16 if bf else torch.float32
        L, d, F, V = dims.n_layers, dims.d_model, dims.d_ff, dims.vocab
        qkv = dims.q_dim + 2 * dims.kv_dim
        dev = torch.device(device)

        def up(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if bf:
                t = t.view(torch.int16).view(torch.bfloat16)
            return t.to(dev)

        def get(name, layer=0):
            if weights is not None:
                return weights[name] if name in ("embed", "lm_head", "final_norm") else weights["layers"][layer][name]
            return synthetic.weight_tensor(dims, name, layer, seed)

        self.embed = up(get("embed"))
        self.lm_head = up(get("lm_head"))
        self.final_norm = up(get("final_norm"))
        self.attn_norm = torch.empty((L, d), dtype=tdt, device=dev)
        self.mlp_norm = torch.empty((L, d), dtype=tdt, device=dev)
        self.wqkv = torch.empty((L, qkv, d), dtype=tdt, device=dev)
        self.wo = torch.empty((L, d, dims.q_dim), dtype=tdt, device=dev)
        self.w_gate_up = torch.empty((L, 2 * F, d), dtype=tdt, device=dev)
        self.w_down = torch.empty((L, d, F), dtype=tdt, device=dev)
        names = ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]
        if threads is None:
            threads = min(16, len(os.sched_getaffinity(0)))

        def layer_arrays(l):
            return {n: get(n, l) for n in names}

        with ThreadPoolExecutor(max(1, threads)) as ex:
            for l, arr in enumerate(ex.map(layer_arrays, range(L))):
                self.attn_norm[l] = up(arr["attn_norm"])
                self.mlp_norm[l] = up(arr["mlp_norm"])
                self.wqkv[l, : dims.q_dim] = up(arr["wq"])
                self.wqkv[l, dims.q_dim: dims.q_dim + dims.kv_dim] = up(arr["wk"])
                self.wqkv[l, dims.q_dim + dims.kv_dim:] = up(arr["wv"])
                self.wo[l] = up(arr["wo"])
                self.w_gate_up[l, :F] = up(arr["w_gate"])
                self.w_gate_up[l, F:] = up(arr["w_up"])
                self.w_down[l] = up(arr["w_down"])
        # the projections in the GEMM's packed layout; the plain copies are dropped
        lib = load()
        dstruct = dims_struct(dims)
        self.packed = torch.empty(lib.la_packed_weight_bytes(C.byref(dstruct)), dtype=torch.uint8, device=dev)
        plain = la_model(*[self.__dict__[n].data_ptr() for n in ("embed", "lm_head", "final_norm", "attn_norm",
                                                                 "wqkv", "wo", "mlp_norm", "w_gate_up", "w_down")],
                         self.packed.data_ptr())
        _check(lib.la_pack_weights(C.byref(dstruct), C.byref(plain), _ptr(self.packed), _stream(None)))
        torch.cuda.synchronize(dev)
        del self.lm_head, self.wqkv, self.wo, self.w_gate_up, self.w_down

    def struct(self) -> la_model:
        return la_model(self.embed.data_ptr(), None, self.final_norm.data_ptr(), self.attn_norm.data_ptr(), None,
                        None, self.mlp_norm.data_ptr(), None, None, self.packed.data_ptr())

    @property
    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.embed, self.final_norm, self.attn_norm, self.mlp_norm,
                                                          self.packed))


# ----------------------------------------------------------------- session


def la_query_sizes(cfg: la_config, dims: la_model_dims) -> la_sizes:
    out = la_sizes()
    _check(load().la_query_sizes(C.byref(cfg), C.byref(dims), C.byref(out)))
    return out


def make_config(W, N, G, max_new, max_prompt, verify_mode=LA_VERIFY_GREEDY, temperature=1.0, seed=0, ar_only=False,
                pool_from_prompt=False, advance_by_accepted=False, cap_full_match=False, pool_from_output=False):
    return la_config(W, N, G, max_new, verify_mode, int(bool(ar_only)), float(temperature), int(seed), max_prompt,
                     int(bool(pool_from_prompt)), int(bool(advance_by_accepted)), int(bool(cap_full_match)),
                     int(bool(pool_from_output)))


class Session:
    """One request: owns its K/V and arena tensors and the library context."""

    def __init__(self, model: DeviceModel, prompt, W, N, G, max_new, verify_mode=LA_VERIFY_GREEDY, temperature=1.0,
                 seed=0, ar_only=False, max_prompt=None, stream=None, pool_from_prompt=False,
                 advance_by_accepted=False, cap_full_match=False, pool_from_output=False):
        lib = load()
        self.model = model
        self.cfg = make_config(W, N, G, max_new, max_prompt or len(prompt), verify_mode, temperature, seed, ar_only,
                               pool_from_prompt, advance_by_accepted, cap_full_match, pool_from_output)
        self.dims = dims_struct(model.dims)
        self.sizes = la_query_sizes(self.cfg, self.dims)
        dev = model.embed.device
        self.kv = torch.empty(int(self.sizes.kv_bytes), dtype=torch.uint8, device=dev)
        self.arena = torch.empty(int(self.sizes.arena_bytes), dtype=torch.uint8, device=dev)
        self.stream = stream
        self._mstruct = model.struct()
        p, pp = _i32(prompt)
        self.ctx = C.c_void_p()
        rc = lib.la_init(C.byref(self.cfg), C.byref(self.dims), C.byref(self._mstruct), _ptr(self.kv),
                         _ptr(self.arena), pp, len(p), _stream(stream), C.byref(self.ctx))
        _check(rc)

    def __del__(self):
        if getattr(self, "ctx", None) and _lib is not None:
            _lib.la_destroy(self.ctx)
            self.ctx = None

    # full rounds ------------------------------------------------------
    def la_step(self):
        buf = (C.c_int32 * LA_MAX_EMIT)()
        n = C.c_int32()
        _check(load().la_step(self.ctx, buf, LA_MAX_EMIT, C.byref(n)), self.ctx)
        return list(buf[: n.value])

    def la_generate(self):
        cap = self.cfg.max_new
        buf = (C.c_int32 * cap)()
        n = C.c_int32()
        _check(load().la_generate(self.ctx, buf, cap, C.byref(n)), self.ctx)
        return list(buf[: n.value])

    # round in steps -----------------------------------------------------
    def la_predict(self) -> la_round_info:
        info = la_round_info()
        _check(load().la_predict(self.ctx, C.byref(info)), self.ctx)
        return info

    def la_verify(self, logits=None, n_inp=0, cand=None):
        """logits: None (pending round) or a device float32 tensor [1 + n_inp + C*S][V]."""
        acc = la_accept()
        z = (C.c_int32 * 128)()
        if logits is None:
            _check(load().la_verify(self.ctx, None, 0, None, 0, C.byref(acc), z), self.ctx)
            return acc, None
        cand = np.zeros((0, self.cfg.N - 1), np.int32) if cand is None else np.asarray(cand, np.int32)
        ca, cp = _i32(cand.reshape(-1))
        _check(load().la_verify(self.ctx, _ptr(logits), int(n_inp), cp, int(len(cand)), C.byref(acc), z), self.ctx)
        return acc, list(z[:n_inp])

    def la_commit(self, acc: la_accept):
        _check(load().la_commit(self.ctx, C.byref(acc)), self.ctx)

    # pool and state -------------------------------------------------------
    def la_pool_lookup(self, key):
        S = self.cfg.N - 1
        out = np.zeros((max(self.cfg.G, 1), S), np.int32)
        n = C.c_int32()
        _check(load().la_pool_lookup(self.ctx, int(key), out.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(n)),
               self.ctx)
        return [tuple(int(t) for t in row) for row in out[: n.value]]

    def la_pool_insert(self, keys, suffixes):
        k, kp = _i32(keys)
        s, sp = _i32(np.asarray(suffixes, np.int32).reshape(-1))
        _check(load().la_pool_insert(self.ctx, kp, sp, len(k)), self.ctx)

    def la_get_state(self, with_window=True, out_cap=None):
        st = la_state_t()
        R = self.cfg.N - 1
        stride = self.cfg.W + self.cfg.N
        win = np.zeros((R, stride), np.int32)
        cap = out_cap or self.cfg.max_new
        outb = np.zeros(cap, np.int32)
        _check(load().la_get_state(self.ctx, C.byref(st), win.ctypes.data_as(C.POINTER(C.c_int32)) if with_window
                                   else None, outb.ctypes.data_as(C.POINTER(C.c_int32)), cap), self.ctx)
        levels = [None if st.level_sizes[r] == 0 else [int(t) for t in win[r, : st.level_sizes[r]]] for r in range(R)]
        return {"round_id": st.round_id, "kv_len": st.kv_len, "n_out": st.n_out, "levels": levels,
                "warm": bool(st.warm), "output": [int(t) for t in outb[: st.n_out]]}

    def la_profile(self, enable=True):
        _check(load().la_profile(self.ctx, int(bool(enable))), self.ctx)

    def la_profile_read(self):
        p = la_profile_t()
        _check(load().la_profile_read(self.ctx, C.byref(p)), self.ctx)
        return {f: getattr(p, f) for f, _ in la_profile_t._fields_}

    def la_stats(self):
        s = la_stats_t()
        _check(load().la_stats(self.ctx, C.byref(s)), self.ctx)
        return {"rounds": s.rounds, "tokens": s.tokens, "candidates": s.candidates, "accepted": s.accepted,
                "hist": list(s.hist), "paused": s.paused}


# ----------------------------------------------------------------- batch


def la_batch_plan(row_budget, S, base_rows, found):
    """The occupancy throttle on host arrays; returns (cap, paused) lists."""
    n = len(base_rows)
    b, bp = _i32(base_rows)
    f, fp = _i32(found)
    cap = np.zeros(max(n, 1), np.int32)
    paused = np.zeros(max(n, 1), np.int32)
    _check(load().la_batch_plan(n, int(row_budget), int(S), bp, fp, cap.ctypes.data_as(C.POINTER(C.c_int32)),
                                paused.ctypes.data_as(C.POINTER(C.c_int32))))
    return [int(x) for x in cap[:n]], [int(x) for x in paused[:n]]


class Batch:
    """Stacked activations for up to max_rows rows of sessions sharing one model (la_batch_*)."""

    def __init__(self, model: DeviceModel, max_rows=256, stream=None):
        lib = load()
        self.model = model
        self.dims = dims_struct(model.dims)
        nbytes = int(lib.la_batch_bytes(C.byref(self.dims), int(max_rows)))
        if nbytes == 0:
            raise LaError(LA_EINVAL, f"max_rows {max_rows} or dims not admitted")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=model.embed.device)
        self._mstruct = model.struct()
        self.max_rows = int(max_rows)
        self.stream = stream
        self.b = C.c_void_p()
        _check(lib.la_batch_init(C.byref(self.dims), C.byref(self._mstruct), int(max_rows), _ptr(self.workspace),
                                 nbytes, _stream(stream), C.byref(self.b)))

    def __del__(self):
        if getattr(self, "b", None) and _lib is not None:
            _lib.la_batch_destroy(self.b)
            self.b = None

    def la_batch_step(self, sessions, row_budget=0):
        """One round of every session; returns (tokens per session, la_batch_round per session)."""
        n = len(sessions)
        ctxs = (C.c_void_p * n)(*[s.ctx for s in sessions])
        buf = np.zeros((n, LA_MAX_EMIT), np.int32)
        nout = np.zeros(n, np.int32)
        info = (la_batch_round * n)()
        _check(load().la_batch_step(self.b, ctxs, n, int(row_budget), buf.ctypes.data_as(C.POINTER(C.c_int32)),
                                    nout.ctypes.data_as(C.POINTER(C.c_int32)), info))
        return [list(map(int, buf[i, : nout[i]])) for i in range(n)], list(info)


# ----------------------------------------------------------------- operators


def rows_desc(p, levels, S, C_, x_t, win_stride, starts=None):
    d = la_rows_desc()
    d.p, d.R, d.C, d.S, d.x_t, d.win_stride = p, len(levels), C_, S, x_t, win_stride
    for r, lv in enumerate(levels):
        d.sizes[r] = 0 if lv is None else len(lv)
        d.starts[r] = 1 if r == 0 else (0 if starts is None else starts[r])
    return d


def la_rows_query(desc: la_rows_desc) -> la_rows_info:
    info = la_rows_info()
    _check(load().la_rows_query(C.byref(desc), C.byref(info)))
    return info


def la_build_rows(desc: la_rows_desc, window_dev, cand_dev, stream=None):
    """Returns (device int32 tensor with the row manifest, la_rows_info)."""
    info = la_rows_query(desc)
    out = torch.empty(info.total_words, dtype=torch.int32, device=window_dev.device)
    _check(load().la_build_rows(C.byref(desc), _ptr(window_dev), _ptr(cand_dev), _ptr(out), _stream(stream),
                                C.byref(info)))
    return out, info


def la_attention(q, k_cache, v_cache, k_ws, v_ws, rows, info, shared_end, out=None, workspace=None, stream=None):
    """Lookahead-mask attention of one layer (device tensors; see include/la.h)."""
    dtype = LA_DTYPE_BF16 if q.dtype == torch.bfloat16 else LA_DTYPE_F32
    Q, H, dh = q.shape
    Hkv, t_cap, _ = k_cache.shape
    ws_cap = k_ws.shape[1] if k_ws is not None else 0
    lib = load()
    need = lib.la_attention_workspace(Q, H, dh, shared_end + info.maxp, t_cap)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(lib.la_attention(dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(k_ws), _ptr(v_ws), ws_cap,
                            H, Hkv, dh, _ptr(rows), C.byref(info), shared_end, _ptr(out), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return out


def la_attention_noalloc(q, k_cache, v_cache, k_ws, v_ws, rows, info, shared_end, out=None, stream=None):
    """la_attention with the library's own split-state array (see include/la.h)."""
    dtype = LA_DTYPE_BF16 if q.dtype == torch.bfloat16 else LA_DTYPE_F32
    Q, H, dh = q.shape
    Hkv, t_cap, _ = k_cache.shape
    ws_cap = k_ws.shape[1] if k_ws is not None else 0
    if out is None:
        out = torch.empty_like(q)
    _check(load().la_attention_noalloc(dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(k_ws), _ptr(v_ws),
                                       ws_cap, H, Hkv, dh, _ptr(rows), C.byref(info), shared_end, _ptr(out),
                                       _stream(stream)))
    return out


def la_linear(epilogue, X, W, R=None, out=None, stream=None):
    """Y = epilogue(X W^T) on device tensors (see include/la.h)."""
    dtype = LA_DTYPE_BF16 if X.dtype == torch.bfloat16 else LA_DTYPE_F32
    M, K = X.shape
    N = W.shape[0] // 2 if epilogue == LA_LINEAR_SWIGLU else W.shape[0]
    lib = load()
    need = lib.la_linear_workspace(dtype, epilogue, M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if epilogue == LA_LINEAR_F32 else X.dtype, device=X.device)
    _check(lib.la_linear(dtype, epilogue, _ptr(X), _ptr(W), _ptr(out), _ptr(R), M, N, K, _ptr(ws), ws.numel(),
                         _stream(stream)))
    return out


def la_pack_linear(epilogue, W, stream=None):
    """Packed copy of an nn.Linear weight (see include/la.h) as a flat uint8 device tensor."""
    dtype = LA_DTYPE_BF16 if W.dtype == torch.bfloat16 else LA_DTYPE_F32
    K = W.shape[1]
    N = W.shape[0] // 2 if epilogue == LA_LINEAR_SWIGLU else W.shape[0]
    lib = load()
    Wp = torch.empty(max(lib.la_packed_linear_bytes(dtype, epilogue, N, K), 1), dtype=torch.uint8, device=W.device)
    _check(lib.la_pack_linear(dtype, epilogue, _ptr(W), N, K, _ptr(Wp), _stream(stream)))
    return Wp


def la_linear_packed(epilogue, X, Wp, N, R=None, out=None, stream=None):
    """la_linear with a weight packed by la_pack_linear (N = output columns)."""
    dtype = LA_DTYPE_BF16 if X.dtype == torch.bfloat16 else LA_DTYPE_F32
    M, K = X.shape
    lib = load()
    need = lib.la_linear_workspace(dtype, epilogue, M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if epilogue == LA_LINEAR_F32 else X.dtype, device=X.device)
    _check(lib.la_linear_packed(dtype, epilogue, _ptr(X), _ptr(Wp), _ptr(out), _ptr(R), M, N, K, _ptr(ws),
                                ws.numel(), _stream(stream)))
    return out
