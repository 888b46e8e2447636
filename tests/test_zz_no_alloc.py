"""The allocation-free attention entry point against la_attention, through the C ABI.

la_attention_noalloc runs la_attention's kernels with the key splits' states in
the library's own device array instead of a caller workspace, so its output
must equal la_attention's bit for bit.  Two calls in a row, the second with a
smaller input (fewer rows, heads and keys), check that the array's leftover
contents from the first call do not leak into the second; an oversized shape
is refused before anything is launched.
"""
import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
la = pytest.importorskip("exact_lookahead_decoding_amd.la")

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.load()


def _case(levels, starts, C, S, p, H, Hkv, dh, seed):
    """Rows built by the library, bf16 inputs (seeded), both entry points."""
    stride = max(len(lv) for lv in levels if lv) + 2
    w = np.zeros((len(levels), stride), np.int32)
    for r, lv in enumerate(levels):
        if lv:
            w[r, : len(lv)] = lv
    cands = np.arange(max(C, 1) * S, dtype=np.int32) % 97
    desc = la.rows_desc(p, levels, S, C, 7, stride, starts)
    rows, info = la.la_build_rows(desc, torch.from_numpy(w).to(DEV), torch.from_numpy(cands).to(DEV))
    Q = info.Q
    g = torch.Generator(device=DEV).manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)  # noqa: E731
    t_cap = p + 16
    q, kc, vc, kw, vw = mk(Q, H, dh), mk(Hkv, t_cap, dh), mk(Hkv, t_cap, dh), mk(Hkv, Q, dh), mk(Hkv, Q, dh)
    print(f"  Q={Q} H={H}/{Hkv} prefix {p}: split state "
          f"{la.load().la_attention_workspace(Q, H, dh, p + info.maxp, t_cap)} bytes", flush=True)
    want = la.la_attention(q, kc, vc, kw, vw, rows, info, p + 1)
    got = la.la_attention_noalloc(q, kc, vc, kw, vw, rows, info, p + 1)
    torch.cuda.synchronize()
    return got, want


def test_noalloc_equals_workspace_path_twice():
    big = ([list(range(100, 115))] * 4, [1, 1, 1, 1], 15, 4, 1024, 32, 32, 128)
    small = ([list(range(100, 104)), list(range(100, 105))], [1, 0], 3, 2, 300, 8, 2, 128)
    for name, (levels, starts, C, S, p, H, Hkv, dh) in (("first", big), ("second, smaller", small)):
        print(f"{name} call", flush=True)
        got, want = _case(levels, starts, C, S, p, H, Hkv, dh, seed=11 if name == "first" else 12)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name


def test_noalloc_refuses_oversized_shape():
    """A shape whose split states exceed the library's array: LA_EOVERFLOW,
    nothing launched (the pointers are never used)."""
    import ctypes as C
    lib = la.load()
    info = la.la_rows_query(la.rows_desc(100, [list(range(14))] + [list(range(15))] * 5, 6, 15, 1, 16,
                                         [1, 0, 0, 0, 0, 0]))
    H, dh, t_cap = 256, 128, 8192
    need = lib.la_attention_workspace(info.Q, H, dh, 8000 + info.maxp, t_cap)
    assert need > la.LA_NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(0x1000)
    rc = lib.la_attention_noalloc(la.LA_DTYPE_BF16, fake, fake, fake, t_cap, fake, fake, info.Q, H, 8, dh,
                                  C.cast(fake, C.POINTER(C.c_int32)), C.byref(info), 8001, fake, None)
    assert rc == la.LA_EOVERFLOW
    assert b"allocation-free" in lib.la_last_error(None)
