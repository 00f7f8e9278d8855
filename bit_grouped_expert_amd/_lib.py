"""ctypes binding of libmoeq4.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes device
tensors (anything with ``data_ptr()``), raw integer addresses or None for NULL.
Every step of the layer runs in the library's HIP kernels; nothing here
computes.  The stream defaults to torch's current stream.  A nonzero status
raises MoEError.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoeq4.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH, \
    MOE_ERR_DEVICE = range(7)


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class moe_shape(C.Structure):
    _fields_ = [("T", C.c_int32), ("d_model", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("d_ff", C.c_int32)]


class moe_q4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("bias", C.c_void_p)]


class moe_q4_ffn(C.Structure):
    _fields_ = [("gate_up", moe_q4), ("down", moe_q4)]


MOE_ENGINE_AUTO, MOE_ENGINE_GROUPED, MOE_ENGINE_RESIDENT, MOE_ENGINE_WIDE, MOE_ENGINE_DECODE = range(5)
ENGINES = {"auto": MOE_ENGINE_AUTO, "grouped": MOE_ENGINE_GROUPED,
           "resident": MOE_ENGINE_RESIDENT, "wide": MOE_ENGINE_WIDE, "decode": MOE_ENGINE_DECODE}
N_STAGE_EVENTS = 6


class moe_layer_opts(C.Structure):
    _fields_ = [("engine", C.c_int32), ("reserved", C.c_int32), ("events", C.POINTER(C.c_void_p))]


class moe_ws_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in
                ("topk_idx", "topk_w", "offsets", "sorted_tok", "slot_row", "act", "y", "sync",
                 "total")]


class moe_layer_plan_info(C.Structure):
    _fields_ = [("gemm_engine", C.c_int32), ("paired", C.c_int32)]


class moe_gqa_shape(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ctx_len", C.c_int32), ("kv_stride", C.c_int64)]


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_workspace_bytes": (C.c_size_t, [C.POINTER(moe_shape)]),
    "moe_workspace_layout": (C.c_int, [C.POINTER(moe_shape), C.POINTER(moe_ws_layout)]),
    "moe_layer_plan": (C.c_int, [C.POINTER(moe_shape), C.c_int32, C.c_int32,
                                 C.POINTER(moe_layer_plan_info)]),
    "moe_grouped_gemm_q4_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32,
                                                         C.c_int32]),
    "moe_route": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                            C.c_void_p, C.c_size_t, C.c_void_p]),
    "moe_route_ex": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_void_p, C.c_float, C.c_void_p, C.c_size_t, C.c_void_p]),
    "moe_permute": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "moe_grouped_gemm_q4": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                      C.c_int32, C.c_void_p, C.c_void_p, moe_q4, C.c_int32,
                                      C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "moe_combine": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_void_p]),
    "moe_layer_forward": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p,
                                    C.POINTER(moe_q4_ffn), C.POINTER(moe_q4_ffn), C.c_void_p,
                                    C.c_void_p, C.c_size_t, C.c_void_p]),
    "moe_layer_forward_ex": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p,
                                       C.POINTER(moe_q4_ffn), C.POINTER(moe_q4_ffn), C.c_void_p,
                                       C.c_void_p, C.c_size_t, C.POINTER(moe_layer_opts),
                                       C.c_void_p]),
    "moe_grouped_gemm_q4_ex": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                         C.c_int32, C.c_void_p, C.c_void_p, moe_q4, C.c_int32,
                                         C.c_void_p, C.c_void_p, C.c_size_t, C.c_int32,
                                         C.c_void_p]),
    "moe_chunked_workspace_bytes": (C.c_size_t, [C.POINTER(moe_shape), C.c_int32]),
    "moe_layer_forward_noalloc": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p,
                                            C.POINTER(moe_q4_ffn), C.POINTER(moe_q4_ffn),
                                            C.c_void_p, C.c_void_p]),
    "moe_layer_forward_chunked": (C.c_int, [C.POINTER(moe_shape), C.c_void_p, C.c_void_p,
                                            C.POINTER(moe_q4_ffn), C.POINTER(moe_q4_ffn),
                                            C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                            C.c_void_p]),
    "moe_gqa_decode_workspace_bytes": (C.c_size_t, [C.POINTER(moe_gqa_shape)]),
    "moe_gqa_decode_attention": (C.c_int, [C.POINTER(moe_gqa_shape), C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                           C.c_void_p]),
}


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_grouped_expert_amd.build` (the HIP path has no fallback)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def shape(T, d_model, n_experts, top_k, d_ff) -> moe_shape:
    return moe_shape(T, d_model, n_experts, top_k, d_ff)


def q4(q, scale, bias) -> moe_q4:
    return moe_q4(_p(q), _p(scale), _p(bias))


def q4_ffn(gate_up: moe_q4, down: moe_q4) -> moe_q4_ffn:
    return moe_q4_ffn(gate_up, down)


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_workspace_bytes(shp: moe_shape) -> int:
    return lib().moe_workspace_bytes(C.byref(shp))


def moe_workspace_layout(shp: moe_shape) -> moe_ws_layout:
    out = moe_ws_layout()
    _check(lib().moe_workspace_layout(C.byref(shp), C.byref(out)), "moe_workspace_layout")
    return out


def moe_layer_plan(shp: moe_shape, engine: str = "auto", has_shared: bool = True) -> moe_layer_plan_info:
    out = moe_layer_plan_info()
    _check(lib().moe_layer_plan(C.byref(shp), ENGINES[engine], int(has_shared), C.byref(out)),
           "moe_layer_plan")
    return out


def moe_grouped_gemm_q4_workspace_bytes(n_groups: int, rows_total: int, a_rows: int, K: int) -> int:
    return lib().moe_grouped_gemm_q4_workspace_bytes(n_groups, rows_total, a_rows, K)


def moe_route(shp, x, router_w, topk_idx, topk_w, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_route(C.byref(shp), _p(x), _p(router_w), _p(topk_idx), _p(topk_w), _p(ws),
                           ws_bytes, _stream(stream)), "moe_route")


def moe_route_ex(shp, x, router_w, topk_idx, topk_w, refine_gap, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_route_ex(C.byref(shp), _p(x), _p(router_w), _p(topk_idx), _p(topk_w),
                              float(refine_gap), _p(ws), ws_bytes, _stream(stream)), "moe_route_ex")


def moe_permute(shp, topk_idx, offsets, sorted_tok, slot_row, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_permute(C.byref(shp), _p(topk_idx), _p(offsets), _p(sorted_tok),
                             _p(slot_row), _p(ws), ws_bytes, _stream(stream)), "moe_permute")


def _engine(engine) -> int:
    return ENGINES[engine] if isinstance(engine, str) else int(engine)


def moe_grouped_gemm_q4(n_groups, rows_total, N, K, A, a_rows, a_row_index, offsets, W: moe_q4,
                        epilogue, Cout, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_grouped_gemm_q4(n_groups, rows_total, N, K, _p(A), a_rows, _p(a_row_index),
                                     _p(offsets), W, epilogue, _p(Cout), _p(ws), ws_bytes,
                                     _stream(stream)), "moe_grouped_gemm_q4")


def moe_grouped_gemm_q4_ex(n_groups, rows_total, N, K, A, a_rows, a_row_index, offsets, W: moe_q4,
                           epilogue, Cout, ws, engine, ws_bytes=None, stream=None):
    """engine: a MOE_ENGINE_* value or one of the names in ENGINES."""
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_grouped_gemm_q4_ex(n_groups, rows_total, N, K, _p(A), a_rows, _p(a_row_index),
                                        _p(offsets), W, epilogue, _p(Cout), _p(ws), ws_bytes,
                                        _engine(engine), _stream(stream)), "moe_grouped_gemm_q4_ex")


def moe_combine(shp, y_sorted, slot_row, topk_w, shared_out, out, stream=None):
    _check(lib().moe_combine(C.byref(shp), _p(y_sorted), _p(slot_row), _p(topk_w), _p(shared_out),
                             _p(out), _stream(stream)), "moe_combine")


def moe_layer_forward(shp, x, router_w, experts: moe_q4_ffn, shared, out, ws, ws_bytes=None,
                      stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    sh = C.byref(shared) if shared is not None else None
    _check(lib().moe_layer_forward(C.byref(shp), _p(x), _p(router_w), C.byref(experts), sh,
                                   _p(out), _p(ws), ws_bytes, _stream(stream)), "moe_layer_forward")


def layer_opts(engine="auto", events=None) -> moe_layer_opts:
    """events: None or a sequence of N_STAGE_EVENTS torch.cuda.Event / raw hipEvent_t ints / None.
    The returned structure keeps the event array alive."""
    o = moe_layer_opts(_engine(engine), 0, None)
    if events is not None:
        raw = (C.c_void_p * N_STAGE_EVENTS)(*[
            None if e is None else (e if isinstance(e, int) else e.cuda_event) for e in events])
        o._events_keep = raw
        o.events = C.cast(raw, C.POINTER(C.c_void_p))
    return o


def moe_layer_forward_ex(shp, x, router_w, experts: moe_q4_ffn, shared, out, ws, opts=None,
                         ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    sh = C.byref(shared) if shared is not None else None
    op = C.byref(opts) if opts is not None else None
    _check(lib().moe_layer_forward_ex(C.byref(shp), _p(x), _p(router_w), C.byref(experts), sh,
                                      _p(out), _p(ws), ws_bytes, op, _stream(stream)),
           "moe_layer_forward_ex")


def moe_chunked_workspace_bytes(shp: moe_shape, chunk_tokens: int) -> int:
    return lib().moe_chunked_workspace_bytes(C.byref(shp), chunk_tokens)


def moe_layer_forward_chunked(shp, x, router_w, experts: moe_q4_ffn, shared, out, chunk_tokens, ws,
                              ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    sh = C.byref(shared) if shared is not None else None
    _check(lib().moe_layer_forward_chunked(C.byref(shp), _p(x), _p(router_w), C.byref(experts), sh,
                                           _p(out), chunk_tokens, _p(ws), ws_bytes,
                                           _stream(stream)), "moe_layer_forward_chunked")


NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_layer_forward_noalloc(shp, x, router_w, experts: moe_q4_ffn, shared, out, stream=None):
    sh = C.byref(shared) if shared is not None else None
    _check(lib().moe_layer_forward_noalloc(C.byref(shp), _p(x), _p(router_w), C.byref(experts), sh,
                                           _p(out), _stream(stream)), "moe_layer_forward_noalloc")


# ---- grouped-query decode attention
def gqa_shape(n_q_heads, n_kv_heads, head_dim, ctx_len, kv_stride=None) -> moe_gqa_shape:
    return moe_gqa_shape(n_q_heads, n_kv_heads, head_dim, ctx_len,
                         ctx_len if kv_stride is None else kv_stride)


def moe_gqa_decode_workspace_bytes(shp: moe_gqa_shape) -> int:
    return lib().moe_gqa_decode_workspace_bytes(C.byref(shp))


def moe_gqa_decode_attention(shp, q, k_cache, v_cache, out, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_gqa_decode_attention(C.byref(shp), _p(q), _p(k_cache), _p(v_cache), _p(out),
                                          _p(ws), ws_bytes, _stream(stream)),
           "moe_gqa_decode_attention")
