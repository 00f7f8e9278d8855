"""C-ABI contract checks that need no GPU: the library loads, exports every entry point
include/moeq4.h declares, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

from bit_grouped_expert_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq4.h")

A = 0x10000          # an aligned fake device address (never dereferenced: every call below fails
B = 0x20000          # validation on the host first)
MIS = 0x10008        # 8-byte aligned only
BIG = 1 << 40


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoeq4.so is not built (python -m bit_grouped_expert_amd.build)")
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L._SIGS), "binding and header disagree"


def test_status_strings(lib):
    for s in range(7):
        assert L.status_string(s)
    assert L.status_string(99) == "unknown status"


def shp(T=512, D=2048, E=256, k=8, F=512):
    return L.shape(T, D, E, k, F)


@pytest.mark.parametrize("bad", [
    dict(T=-1), dict(D=0), dict(D=100), dict(F=96), dict(E=0), dict(E=1025), dict(k=0),
    dict(k=33), dict(E=4, k=5), dict(T=1 << 20), dict(T=100000, D=4096),
])
def test_shape_rules(lib, bad):
    s = shp(**bad)
    assert L.moe_workspace_bytes(s) == 0
    assert lib.moe_layer_forward(C.byref(s), A, A, C.byref(L.moe_q4_ffn()), None, A, A, BIG, None) \
        == L.MOE_ERR_SHAPE
    assert lib.moe_route(C.byref(s), A, A, A, A, A, BIG, None) == L.MOE_ERR_SHAPE


def test_workspace_bytes_monotone_and_layout(lib):
    prev = 0
    for T in [0, 1, 4, 16, 255, 256, 257, 512, 4096, 8192, 32768]:
        s = shp(T=T)
        n = L.moe_workspace_bytes(s)
        assert n >= prev
        prev = n
        lay = L.moe_workspace_layout(s)
        offs = [lay.topk_idx, lay.topk_w, lay.offsets, lay.sorted_tok, lay.slot_row, lay.act, lay.y]
        assert all(o % 256 == 0 for o in offs)
        assert offs == sorted(offs) and lay.total == n
        assert lay.y + (9 * T) * 2048 * 2 <= n
        # the counters of the persistent launches: one word per tile past the first 64
        assert lay.sync % 256 == 0 and lay.sync >= lay.y + (9 * T) * 2048 * 2
        assert lay.sync + 4 * (64 + (9 * T) // 32 + 257) <= n
    assert L.moe_grouped_gemm_q4_workspace_bytes(0, 10, 10, 64) == 0
    assert L.moe_grouped_gemm_q4_workspace_bytes(4, 10, 10, 96) == 0       # K % 64 != 0
    assert L.moe_grouped_gemm_q4_workspace_bytes(4, 10, -1, 64) == 0
    need = L.moe_grouped_gemm_q4_workspace_bytes(257, 4608, 512, 2048)
    assert need >= (4608 // 32 + 257) * 16 + 512 * 32 * 4       # tile map + row sums of A
    assert L.moe_grouped_gemm_q4_workspace_bytes(257, 4608, 1024, 2048) > need


def test_layer_plan(lib):
    """The engine and launch shape the layer calls take (host-only; without a GPU the
    compute-unit count defaults to 256)."""
    p = L.moe_layer_plan(shp(T=512))
    assert (p.gemm_engine, p.paired) == (L.MOE_ENGINE_RESIDENT, 1)
    p = L.moe_layer_plan(shp(T=8192))
    assert (p.gemm_engine, p.paired) == (L.MOE_ENGINE_WIDE, 0)
    assert L.moe_layer_plan(shp(T=1)).gemm_engine == L.MOE_ENGINE_DECODE
    p = L.moe_layer_plan(shp(T=1), "resident")
    assert (p.gemm_engine, p.paired) == (L.MOE_ENGINE_RESIDENT, 1)
    p = L.moe_layer_plan(shp(T=512), "grouped")
    assert (p.gemm_engine, p.paired) == (L.MOE_ENGINE_GROUPED, 0)
    # d_ff = 128: no resident plan (K = F must be a multiple of 256)
    assert L.moe_layer_plan(shp(T=512, F=128)).gemm_engine == L.MOE_ENGINE_GROUPED
    with pytest.raises(L.MoEError):
        L.moe_layer_plan(shp(T=512, F=128), "resident")
    with pytest.raises(L.MoEError):
        L.moe_layer_plan(shp(T=512), "decode")


def ffn(q=A, s=A, b=A):
    return L.q4_ffn(L.q4(q, s, b), L.q4(q, s, b))


def test_layer_forward_validation(lib):
    s = shp()
    need = L.moe_workspace_bytes(s)
    e, sh = ffn(), ffn()
    f = lambda *a: lib.moe_layer_forward(*a)  # noqa: E731
    assert f(None, A, A, C.byref(e), C.byref(sh), A, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), 0, A, C.byref(e), C.byref(sh), A, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), A, A, None, C.byref(sh), A, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), A, A, C.byref(ffn(s=0)), C.byref(sh), A, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), A, A, C.byref(e), C.byref(ffn(b=0)), A, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), A, A, C.byref(e), C.byref(sh), 0, A, need, None) == L.MOE_ERR_NULL
    assert f(C.byref(s), MIS, A, C.byref(e), C.byref(sh), A, A, need, None) == L.MOE_ERR_ALIGN
    assert f(C.byref(s), A, A, C.byref(ffn(q=MIS)), C.byref(sh), A, A, need, None) == L.MOE_ERR_ALIGN
    assert f(C.byref(s), A, A, C.byref(e), C.byref(sh), A, 0, need, None) == L.MOE_ERR_WORKSPACE
    assert f(C.byref(s), A, A, C.byref(e), C.byref(sh), A, A, need - 1, None) == L.MOE_ERR_WORKSPACE
    assert f(C.byref(s), A, A, C.byref(e), C.byref(sh), A, MIS, need, None) == L.MOE_ERR_ALIGN
    # T = 0 is a no-op (returns before touching the device)
    s0 = shp(T=0)
    assert f(C.byref(s0), 0, 0, None, None, 0, 0, 0, None) == L.MOE_OK


def test_route_permute_combine_validation(lib):
    s = shp()
    need = L.moe_workspace_bytes(s)
    assert lib.moe_route(C.byref(s), A, 0, A, A, A, need, None) == L.MOE_ERR_NULL
    assert lib.moe_route(C.byref(s), A, A, MIS, A, A, need, None) == L.MOE_ERR_ALIGN
    assert lib.moe_route(C.byref(s), A, A, A, A, A, need - 1, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_route_ex(C.byref(s), A, A, A, A, -1.0, A, need, None) == L.MOE_ERR_SHAPE
    assert lib.moe_route_ex(C.byref(s), A, A, A, A, float("nan"), A, need, None) == L.MOE_ERR_SHAPE
    assert lib.moe_permute(C.byref(s), 0, A, A, A, A, need, None) == L.MOE_ERR_NULL
    assert lib.moe_permute(C.byref(s), A, A, MIS, A, A, need, None) == L.MOE_ERR_ALIGN
    assert lib.moe_permute(C.byref(s), A, A, A, A, None, need, None) == L.MOE_ERR_WORKSPACE
    s0 = shp(T=0)       # empty routing: only the offsets are required
    assert lib.moe_permute(C.byref(s0), None, None, None, None, A, need, None) == L.MOE_ERR_NULL
    assert lib.moe_permute(C.byref(s0), None, MIS, None, None, A, need, None) == L.MOE_ERR_ALIGN
    assert lib.moe_combine(C.byref(s), A, 0, A, None, A, None) == L.MOE_ERR_NULL
    assert lib.moe_combine(C.byref(s), A, A, A, MIS, A, None) == L.MOE_ERR_ALIGN
    assert lib.moe_combine(C.byref(shp(D=65)), A, A, A, None, A, None) == L.MOE_ERR_SHAPE


def test_grouped_gemm_validation(lib):
    W = L.q4(A, A, A)
    need = L.moe_grouped_gemm_q4_workspace_bytes(4, 100, 100, 256)
    g = lambda n_groups=4, rows=100, N=128, K=256, Ap=A, a_rows=100, idx=None, off=A, w=W, ep=0, \
        Cp=B, ws=A, wsb=need: lib.moe_grouped_gemm_q4(n_groups, rows, N, K, Ap, a_rows, idx, off, w,  # noqa
                                                     ep, Cp, ws, wsb, None)
    assert g(n_groups=0) == L.MOE_ERR_SHAPE
    assert g(N=96) == L.MOE_ERR_SHAPE
    assert g(K=100) == L.MOE_ERR_SHAPE
    assert g(ep=2) == L.MOE_ERR_SHAPE
    assert g(rows=-1) == L.MOE_ERR_SHAPE
    assert g(rows=1 << 25, N=128) == L.MOE_ERR_SHAPE
    assert g(rows=0) == L.MOE_OK          # nothing to do, nothing enqueued
    assert g(Ap=0) == L.MOE_ERR_NULL
    assert g(off=0) == L.MOE_ERR_NULL
    assert g(w=L.q4(A, 0, A)) == L.MOE_ERR_NULL
    assert g(Cp=0) == L.MOE_ERR_NULL
    assert g(Ap=MIS) == L.MOE_ERR_ALIGN
    assert g(idx=MIS) == L.MOE_ERR_ALIGN
    assert g(w=L.q4(A, A, MIS)) == L.MOE_ERR_ALIGN
    assert g(ws=0) == L.MOE_ERR_WORKSPACE
    assert g(wsb=need - 1) == L.MOE_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.lib()


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """moe_layer_forward_noalloc checks the shape's workspace against its static scratch on the
    host, before any HIP call: 1024 tokens of the 2048/256/8/512 layer need 53.6 MiB."""
    big = shp(T=1024)
    assert L.moe_workspace_bytes(big) > L.NOALLOC_SCRATCH_BYTES
    q = L.q4(A, A, A)
    ffn = L.q4_ffn(q, q)
    assert lib.moe_layer_forward_noalloc(C.byref(big), A, A, C.byref(ffn), C.byref(ffn), A, None) \
        == L.MOE_ERR_WORKSPACE
    assert L.moe_workspace_bytes(shp(T=512)) <= L.NOALLOC_SCRATCH_BYTES
    bad = shp(D=100)
    assert lib.moe_layer_forward_noalloc(C.byref(bad), A, A, C.byref(ffn), None, A, None) \
        == L.MOE_ERR_SHAPE


@pytest.mark.parametrize("bad", [(16, 2, 64, 100, 100), (16, 3, 128, 100, 100), (34, 2, 128, 100, 100),
                                 (16, 2, 128, 0, 0), (16, 2, 128, 100, 99), (16, 0, 128, 1, 1)])
def test_gqa_attention_shape_rules(lib, bad):
    """Unsupported attention shapes: zero workspace and MOE_ERR_SHAPE before any HIP call
    (head dim other than 128, query heads not a multiple of KV heads, more than 16 per KV head,
    an empty cache, a stride shorter than the cache, no KV head)."""
    shp = L.moe_gqa_shape(*bad)
    assert lib.moe_gqa_decode_workspace_bytes(C.byref(shp)) == 0
    st = lib.moe_gqa_decode_attention(C.byref(shp), A, A, A, A, A, BIG, None)
    assert st == L.MOE_ERR_SHAPE


def test_gqa_attention_validation(lib):
    shp = L.gqa_shape(16, 2, 128, 32768)
    need = lib.moe_gqa_decode_workspace_bytes(C.byref(shp))
    assert need >= 2 * 256 * 8 * 130 * 4
    call = lambda q=A, k=A, v=A, o=A, ws=A, n=need: lib.moe_gqa_decode_attention(
        C.byref(shp), q, k, v, o, ws, n, None)
    assert call(q=None) == L.MOE_ERR_NULL
    assert call(ws=None) == L.MOE_ERR_NULL
    assert call(k=MIS) == L.MOE_ERR_ALIGN
    assert call(n=need - 1) == L.MOE_ERR_WORKSPACE
