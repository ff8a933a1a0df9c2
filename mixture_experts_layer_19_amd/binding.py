"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function here has the name of the C entry point it calls and passes
device pointers (torch tensors' ``data_ptr()``), sizes and stream handles
through unchanged.  All arithmetic happens in the HIP kernels.  Loading
fails loudly if ``libmoe.so`` has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8, MOE_MXFP4, MOE_FP8 = 0, 1, 2, 3, 4
MOE_WS_ROUTE, MOE_WS_PERMUTE, MOE_WS_GROUPED_FFN, MOE_WS_SHARED_FFN, MOE_WS_LAYER = range(5)
MOE_PACK_GATE_UP, MOE_PACK_DOWN, MOE_PACK_GATE_UP_SCALE, MOE_PACK_DOWN_SCALE = range(4)

# every symbol include/moe.h declares
EXPORTS = ("moe_ctx_create", "moe_ctx_destroy", "moe_status_string", "moe_ctx_last_error",
           "moe_workspace_bytes", "moe_packed_bytes", "moe_pack_experts", "moe_mx_quantize",
           "moe_fp8_quantize",
           "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_ws_topk", "moe_ctx_set_profiling", "moe_ctx_stage_ms",
           "moe_layer_forward_noalloc")
STAGES = ("route", "mx_quant", "permute", "gate_up", "down", "shared_gate_up", "shared_down",
          "combine")


class MoeDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("router_scaling_factor", ctypes.c_float),
                ("route_norm", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("fp8_x_scale", ctypes.c_float), ("fp8_h_scale", ctypes.c_float),
                ("fp8_sh_h_scale", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "gate_up", "down", "gate_up_scale", "down_scale",
        "sh_gate_up", "sh_down", "sh_gate_up_scale", "sh_down_scale")]


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_lock = threading.Lock()
_lib = None


def lib():
    """Load libmoe.so (raises if it is missing: build it first)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        DP, WP = ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeWeights)
        sig = {
            "moe_ctx_create": ([ctypes.c_int, P, ctypes.POINTER(P)], ctypes.c_int),
            "moe_ctx_destroy": ([P], ctypes.c_int),
            "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "moe_ctx_last_error": ([P], ctypes.c_char_p),
            "moe_workspace_bytes": ([DP, I32, ctypes.c_int], S),
            "moe_packed_bytes": ([DP, ctypes.c_int, ctypes.c_int], S),
            "moe_pack_experts": ([DP, ctypes.c_int, ctypes.c_int] + [P] * 8, ctypes.c_int),
            "moe_mx_quantize": ([P, ctypes.c_int, I64, I64, P, P, P], ctypes.c_int),
            "moe_fp8_quantize": ([P, ctypes.c_int, I64, ctypes.c_float, P, P], ctypes.c_int),
            "moe_route": ([P, DP, P, I32, P, P, P, P, P, S, P], ctypes.c_int),
            "moe_permute": ([P, DP, P, I32, P, P, P, P, P, S, P], ctypes.c_int),
            "moe_grouped_ffn": ([P, DP, WP, ctypes.c_int, P, I32, P, P, P, P, S, P], ctypes.c_int),
            "moe_combine": ([P, DP, P, P, P, P, I32, P, P], ctypes.c_int),
            "moe_layer_forward": ([P, DP, WP, P, I32, P, P, S, P], ctypes.c_int),
            "moe_layer_forward_noalloc": ([P, DP, WP, P, I32, P, P], ctypes.c_int),
            "moe_layer_ws_topk": ([DP, I32, ctypes.POINTER(S), ctypes.POINTER(S)], ctypes.c_int),
            "moe_ctx_set_profiling": ([P, ctypes.c_int], ctypes.c_int),
            "moe_ctx_stage_ms": ([P, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
        return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc, ctx=None):
    if rc != MOE_OK:
        L = lib()
        msg = L.moe_status_string(rc).decode()
        if ctx is not None:
            extra = L.moe_ctx_last_error(ctx).decode()
            if extra:
                msg += ": " + extra
        raise MoeError(rc, msg)


# ----------------------------------------------------------------------------- entry points


def moe_ctx_create(device: int, side_stream=None):
    h = ctypes.c_void_p()
    _check(lib().moe_ctx_create(device, _stream(side_stream), ctypes.byref(h)))
    return h.value


def moe_ctx_destroy(ctx):
    _check(lib().moe_ctx_destroy(ctx))


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_workspace_bytes(desc: MoeDesc, T: int, which: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(desc), T, which)


def moe_packed_bytes(desc: MoeDesc, shared: int, which: int) -> int:
    return lib().moe_packed_bytes(ctypes.byref(desc), shared, which)


def moe_pack_experts(desc, shared, src_dtype, gate, up, down, gate_up_out, down_out,
                     gate_up_scale_out=None, down_scale_out=None, stream=None):
    _check(lib().moe_pack_experts(ctypes.byref(desc), shared, src_dtype, _ptr(gate), _ptr(up),
                                  _ptr(down), _ptr(gate_up_out), _ptr(down_out),
                                  _ptr(gate_up_scale_out), _ptr(down_scale_out), _stream(stream)))


def moe_mx_quantize(src, src_dtype, rows, cols, q, scale, stream=None):
    _check(lib().moe_mx_quantize(_ptr(src), src_dtype, rows, cols, _ptr(q), _ptr(scale),
                                 _stream(stream)))


def moe_fp8_quantize(src, src_dtype, n, scale, q, stream=None):
    _check(lib().moe_fp8_quantize(_ptr(src), src_dtype, n, scale, _ptr(q), _stream(stream)))


def moe_route(ctx, desc, x, T, router_w, router_bias, topk_idx, topk_w, ws, ws_bytes,
              stream=None):
    _check(lib().moe_route(ctx, ctypes.byref(desc), _ptr(x), T, _ptr(router_w), _ptr(router_bias),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)), ctx)


def moe_permute(ctx, desc, topk_idx, T, counts, offsets, sorted_src, dest, ws, ws_bytes,
                stream=None):
    _check(lib().moe_permute(ctx, ctypes.byref(desc), _ptr(topk_idx), T, _ptr(counts),
                             _ptr(offsets), _ptr(sorted_src), _ptr(dest), _ptr(ws), ws_bytes,
                             _stream(stream)), ctx)


def moe_grouped_ffn(ctx, desc, weights, shared, x, T, sorted_src, offsets, y, ws, ws_bytes,
                    stream=None):
    _check(lib().moe_grouped_ffn(ctx, ctypes.byref(desc), ctypes.byref(weights), shared, _ptr(x),
                                 T, _ptr(sorted_src), _ptr(offsets), _ptr(y), _ptr(ws), ws_bytes,
                                 _stream(stream)), ctx)


def moe_combine(ctx, desc, y, dest, topk_w, shared_out, T, out, stream=None):
    _check(lib().moe_combine(ctx, ctypes.byref(desc), _ptr(y), _ptr(dest), _ptr(topk_w),
                             _ptr(shared_out), T, _ptr(out), _stream(stream)), ctx)


def moe_layer_forward(ctx, desc, weights, x, T, out, ws, ws_bytes, stream=None):
    _check(lib().moe_layer_forward(ctx, ctypes.byref(desc), ctypes.byref(weights), _ptr(x), T,
                                   _ptr(out), _ptr(ws), ws_bytes, _stream(stream)), ctx)


def moe_layer_forward_noalloc(ctx, desc, weights, x, T, out, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctx, ctypes.byref(desc), ctypes.byref(weights),
                                           _ptr(x), T, _ptr(out), _stream(stream)), ctx)


# bytes of the static workspace moe_layer_forward_noalloc uses (include/moe.h)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_ws_topk(desc, T):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_layer_ws_topk(ctypes.byref(desc), T, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def moe_ctx_set_profiling(ctx, enable: bool):
    _check(lib().moe_ctx_set_profiling(ctx, int(bool(enable))), ctx)


def moe_ctx_stage_ms(ctx) -> dict:
    arr = (ctypes.c_float * len(STAGES))()
    _check(lib().moe_ctx_stage_ms(ctx, arr), ctx)
    return dict(zip(STAGES, (float(v) for v in arr)))
