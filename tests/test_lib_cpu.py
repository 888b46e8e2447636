"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
symbol include/la.h declares, sizes rounds like the oracle, rejects bad input."""
import os
import re

import pytest

import synthetic
from conftest import ROOT
from oracle import rows as orows

la = pytest.importorskip("exact_lookahead_decoding_amd.la")


def _lib():
    try:
        return la.load()
    except RuntimeError as e:
        pytest.fail(f"library not built: {e}")


def test_exports_match_header():
    lib = _lib()
    hdr = open(os.path.join(ROOT, "include", "la.h")).read()
    names = set(re.findall(r"^\s*(?:int|void|size_t|uint64_t|const char\*)\s+(la_\w+)\s*\(", hdr, flags=re.M))
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(la.EXPORTS) == names


@pytest.mark.parametrize("W,N,G,q", [(7, 5, 7, 56), (15, 5, 15, 120), (5, 3, 5, 20), (15, 7, 15, 180), (5, 4, 2, 21)])
def test_query_sizes_row_ledger(W, N, G, q):
    d = la.dims_struct(synthetic.PRESETS["llama7b"])
    s = la.la_query_sizes(la.make_config(W, N, G, 64, 100), d)
    assert s.q_max == q == (W + G) * (N - 1)
    assert s.kv_bytes == 2 * 32 * 32 * s.t_cap * 128 * 2


def test_invalid_configs_rejected():
    d = la.dims_struct(synthetic.PRESETS["tiny"])
    for args in [(5, 2, 5), (5, 1, 5), (0, 3, 5), (5, 3, -1), (5, 17, 5)]:
        with pytest.raises(la.LaError) as e:
            la.la_query_sizes(la.make_config(*args, 10, 10), d)
        assert e.value.code == la.LA_EINVAL


def test_option_flags_validated():
    """pool_from_prompt, advance_by_accepted, cap_full_match and pool_from_output are 0 or 1."""
    d = la.dims_struct(synthetic.PRESETS["tiny"])
    la.la_query_sizes(la.make_config(5, 3, 5, 10, 10, pool_from_prompt=True, advance_by_accepted=True,
                                     cap_full_match=True, pool_from_output=True), d)
    for field in ("pool_from_prompt", "advance_by_accepted", "cap_full_match", "pool_from_output"):
        cfg = la.make_config(5, 3, 5, 10, 10)
        setattr(cfg, field, 2)
        with pytest.raises(la.LaError) as e:
            la.la_query_sizes(cfg, d)
        assert e.value.code == la.LA_EINVAL, field


def test_attention_rejects_bad_arguments():
    """Host-side validation of la_attention: every case below is refused before
    anything is launched (the pointers are never dereferenced)."""
    import ctypes as C
    lib = _lib()
    info = la.la_rows_query(la.rows_desc(100, [list(range(4)), list(range(5))], 2, 2, 1, 8, [1, 0]))
    fake = C.c_void_p(0x1000)
    rows = C.cast(fake, C.POINTER(C.c_int32))
    Q, H, Hkv, dh, t_cap = info.Q, 4, 2, 64, 256
    need = lib.la_attention_workspace(Q, H, dh, 100 + info.maxp, t_cap)

    def call(dtype=la.LA_DTYPE_BF16, q=fake, H=H, Hkv=Hkv, shared_end=101, ws_bytes=need, t_cap=t_cap):
        return lib.la_attention(dtype, q, fake, fake, t_cap, fake, fake, Q, H, Hkv, dh, rows, C.byref(info),
                                shared_end, fake, fake, ws_bytes, None)
    assert call(q=None) == la.LA_EINVAL                   # null argument
    assert call(dtype=7) == la.LA_EINVAL                  # unknown dtype
    assert call(H=5) == la.LA_EINVAL                      # H not a multiple of Hkv
    assert call(shared_end=0) == la.LA_EINVAL             # nothing committed
    assert call(shared_end=t_cap + 1) == la.LA_EINVAL     # past the cache
    assert call(ws_bytes=need - 1) == la.LA_EOVERFLOW     # workspace too small


def test_build_rows_rejects_oversized_window():
    """More window columns than the row builder's tables hold: refused before any launch."""
    import ctypes as C
    lib = _lib()
    desc = la.rows_desc(100, [list(range(200)), None], 2, 0, 1, 256, [1, 0])
    info = la.la_rows_info()
    fake = C.c_void_p(0x1000)
    rc = lib.la_build_rows(C.byref(desc), C.cast(fake, C.POINTER(C.c_int32)), C.cast(fake, C.POINTER(C.c_int32)),
                           C.cast(fake, C.POINTER(C.c_int32)), None, C.byref(info))
    assert rc == la.LA_EOVERFLOW


def _oracle_layout(levels, starts, C, S):
    cands = [tuple(range(S)) for _ in range(C)]
    return orows.compile_round(1, 10, levels, cands, S, starts=starts)


@pytest.mark.parametrize("sizes,starts,C,S", [
    ([4, 5, 5], [1, 0, 0], 2, 3),
    ([6, 0, 0], [1, 0, 0], 0, 3),
    ([5, 6, 0], [1, 0, 0], 0, 3),
    ([15, 15, 15, 15], [1, 1, 1, 1], 15, 4),
    ([14, 15, 15, 15, 15, 15], [1, 0, 0, 0, 0, 0], 15, 6),
    ([0, 0], [1, 0], 0, 2),
])
def test_rows_query_matches_oracle(sizes, starts, C, S):
    levels = [None if n == 0 else list(range(n)) for n in sizes]
    comp = _oracle_layout(levels, starts, C, S)
    info = la.la_rows_query(la.rows_desc(10, levels, S, C, 1, 32, starts))
    assert info.Q == comp.Q
    assert info.n_inp == len(comp.inp)
    assert info.n_logit == 1 + len(comp.inp) + len(comp.guess)


@pytest.mark.parametrize("W,N,G,why", [
    (40, 8, 5, "rows"),        # (W + G) * (N - 1) = 315 packed rows: above one GEMM launch's 256
    (60, 10, 5, "rows"),       # 585 rows
    (62, 3, 64, "stage"),      # 252 rows: under 256, but beyond the tail stage
    (64, 4, 0, "reach"),       # 192 rows, but the first warmup fill's last column reaches 65 positions
    (63, 4, 0, None),          # 189 rows, 64 positions: admitted
    (15, 7, 15, None),         # the 34B-shaped workload: 180 rows
    (36, 6, 5, None),          # 205 rows: the attention's tail stage still holds them at head dim 128
    (30, 8, 0, None),          # 210 rows
    (38, 6, 5, "stage"),       # 215 rows: it does not
    (20, 7, 20, "stage"),      # 240 rows
])
def test_round_shapes_admitted_before_state(W, N, G, why):
    """A config whose largest round exceeds what the round's kernels take is
    refused by la_query_sizes (and la_init) with LA_EINVAL, before any state
    exists ("M7.3", 0x01A admission), instead of failing at its first warm
    round: more than 256 packed rows (one GEMM launch), a branch reaching
    more than 64 positions past the committed prefix (the attention's path
    table), or more rows than the attention's tail stage holds in LDS (the
    committed part of the first tail chunk, every packed row's K and V and
    the branch path table beside two ring slots: about 210 rows at head dim
    128 in bf16)."""
    d = la.dims_struct(synthetic.PRESETS["llama7b"])
    cfg = la.make_config(W, N, G, 64, 100)
    rows = (W + G) * (N - 1)
    if why is None:
        s = la.la_query_sizes(cfg, d)
        assert s.q_max == rows
        return
    with pytest.raises(la.LaError) as e:
        la.la_query_sizes(cfg, d)
    assert e.value.code == la.LA_EINVAL
    msg = str(e.value)
    want = {"rows": "at most 256", "reach": "positions past", "stage": "tail stage"}[why]
    assert want in msg, msg


def test_d_model_bound_admitted():
    """The embedding gather and the residual-fold RMSNorm hold a row in 2048
    16-byte vectors: bf16 d_model up to 16384, fp32 up to 8192."""
    import dataclasses
    base = synthetic.PRESETS["llama7b"]
    cfg = la.make_config(7, 5, 7, 64, 100)
    la.la_query_sizes(cfg, la.dims_struct(dataclasses.replace(base, d_model=16384)))
    with pytest.raises(la.LaError) as e:
        la.la_query_sizes(cfg, la.dims_struct(dataclasses.replace(base, d_model=16384 + 128)))
    assert e.value.code == la.LA_EINVAL
    f32 = dataclasses.replace(base, dtype="f32", d_model=8192 + 64)
    with pytest.raises(la.LaError) as e:
        la.la_query_sizes(cfg, la.dims_struct(f32))
    assert e.value.code == la.LA_EINVAL
