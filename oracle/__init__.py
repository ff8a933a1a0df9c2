"""CPU oracle for one Hunyuan-style MoE layer forward pass -- TEST INFRASTRUCTURE.

This package is the plain, slow, obviously correct reference that the GPU
library is checked against.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the GPU library never does, and
this package imports nothing from the GPU library.

The arithmetic lives in ``moe_oracle.c`` (plain C, double accumulation in a
fixed order, OpenMP across independent rows).  This module builds it with gcc,
loads it with ctypes and exposes numpy-level wrappers.  The per-token
composition in :func:`layer_forward_tokens` follows the definition of the
layer output directly: for a token t,

    out[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t])  +  FFN_shared(x[t])

(Hy3 on CANN NPU guide, section 1 and section 8.5; HunyuanImage-3.0
multi-stream article, source walkthrough part 3), which lets a test check
sampled rows of a full-size layer without running the whole oracle.

Parity pins for every function here are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_mxq.argtypes = [I64, P, P, P]
        lib.oracle_mx_dequant.argtypes = [I64, P, P, P]
        lib.oracle_e2m1_decode.restype = ctypes.c_double
        lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        lib.oracle_mxq4.argtypes = [I64, P, P, P]
        lib.oracle_fp8_tensor_scale.restype = ctypes.c_float
        lib.oracle_fp8_tensor_scale.argtypes = [I64, P]
        lib.oracle_fp8_quantize.argtypes = [I64, P, ctypes.c_float, P]
        lib.oracle_swiglu_rows_fp8.argtypes = [I64, I64, I64, P, P, P, P, ctypes.c_float,
                                               ctypes.c_float, P, P]
        lib.oracle_mx4_dequant.argtypes = [I64, P, P, P]
        lib.oracle_router_logits.argtypes = [I64, I64, I64, P, P, P, P]
        lib.oracle_route.argtypes = [I64, I64, I64, I64, P, P, P, ctypes.c_float, ctypes.c_int,
                                     P, P, P, P]
        lib.oracle_route_weights.argtypes = [I64, I64, I64, P, P, ctypes.c_float, ctypes.c_int, P]
        lib.oracle_permute.argtypes = [I64, I64, I64, P, P, P, P, P]
        lib.oracle_swiglu_rows.argtypes = [I64, I64, I64, P, ctypes.c_int, P, P, P, ctypes.c_int,
                                           P, P]
        lib.oracle_combine.argtypes = [I64, I64, I64, P, P, P, P, P]
        lib.oracle_layer_forward.argtypes = (
            [I64, I64, I64, I64, I64, I64, ctypes.c_float, ctypes.c_int, P, P, P, ctypes.c_int]
            + [P] * 6 + [ctypes.c_int] + [P] * 10)
        for name in ("oracle_mxq", "oracle_mx_dequant", "oracle_mxq4", "oracle_mx4_dequant",
                     "oracle_fp8_quantize", "oracle_swiglu_rows_fp8",
                     "oracle_router_logits", "oracle_route", "oracle_route_weights",
                     "oracle_permute", "oracle_swiglu_rows", "oracle_combine",
                     "oracle_layer_forward"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _weights(w):
    """Weights are fp32 arrays or bf16 bit patterns (uint16 arrays)."""
    w = np.ascontiguousarray(w)
    if w.dtype == np.uint16:
        return w, 1
    return np.ascontiguousarray(w, dtype=np.float32), 0


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------------------- MX-fp8


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def mxq(v):
    """MX-fp8 quantisation along the last axis (length a multiple of 32).
    Returns (codes uint8, same shape; scales uint8, last axis / 32)."""
    v = _f32(v)
    if v.shape[-1] % 32:
        raise ValueError("last axis must be a multiple of 32")
    nblk = v.size // 32
    q = np.empty(v.shape, np.uint8)
    s = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    _check(_load().oracle_mxq(nblk, _p(v), _p(q), _p(s)), "mxq")
    return q, s


def mx_dequant(q, s):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    v = np.empty(q.shape, np.float32)
    _check(_load().oracle_mx_dequant(q.size // 32, _p(q), _p(s), _p(v)), "mx_dequant")
    return v


# ----------------------------------------------------------------------------- MXFP4

# MX modes of the FFN and layer functions: none, MX-fp8 experts and
# activations (W8A8), MXFP4 routed experts with MX-fp8 activations (W4A8;
# the shared expert stays W8A8)
MX_NONE, MX_FP8, MX_W4A8 = 0, 1, 2


def e2m1_decode(code: int) -> float:
    return _load().oracle_e2m1_decode(int(code))


def e2m1_encode(v: float) -> int:
    return int(_load().oracle_e2m1_encode(float(v)))


def mxq4(v):
    """MXFP4 quantisation along the last axis (length a multiple of 32).
    Returns (codes uint8 in 0..15, one per element; scales uint8, last axis / 32)."""
    v = _f32(v)
    if v.shape[-1] % 32:
        raise ValueError("last axis must be a multiple of 32")
    q = np.empty(v.shape, np.uint8)
    s = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    _check(_load().oracle_mxq4(v.size // 32, _p(v), _p(q), _p(s)), "mxq4")
    return q, s


def mx4_dequant(q, s):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    v = np.empty(q.shape, np.float32)
    _check(_load().oracle_mx4_dequant(q.size // 32, _p(q), _p(s), _p(v)), "mx4_dequant")
    return v


# ----------------------------------------------------------------------------- static FP8


def fp8_tensor_scale(w) -> float:
    """Per-tensor weight scale fp32(max|w| / 448) (1 for an all-zero tensor)."""
    w = _f32(w)
    return float(_load().oracle_fp8_tensor_scale(w.size, _p(w)))


def fp8_quantize(v, s):
    """E4M3 codes of fp32(v / s) (round to nearest even, saturating)."""
    v = _f32(v)
    q = np.empty(v.shape, np.uint8)
    _check(_load().oracle_fp8_quantize(v.size, _p(v), ctypes.c_float(s), _p(q)), "fp8_quantize")
    return q


def swiglu_rows_fp8(xrows, Wg, Wu, Wd, s_x, s_h):
    """One expert's SwiGLU FFN with static per-tensor FP8 (fp32 masters in;
    weight scales from fp8_tensor_scale, activation scales s_x and s_h).
    Returns (h [M,I] before quantisation, y [M,H])."""
    xrows = _f32(xrows)
    M, H = xrows.shape
    Wg, Wu, Wd = _f32(Wg), _f32(Wu), _f32(Wd)
    I = Wg.shape[0]
    h = np.empty((M, I), np.float32)
    y = np.empty((M, H), np.float32)
    _check(_load().oracle_swiglu_rows_fp8(M, H, I, _p(xrows), _p(Wg), _p(Wu), _p(Wd),
                                          ctypes.c_float(s_x), ctypes.c_float(s_h), _p(h), _p(y)),
           "swiglu_rows_fp8")
    return h, y


def _mx_mode(mx) -> int:
    m = int(mx)
    if m not in (MX_NONE, MX_FP8, MX_W4A8):
        raise ValueError("mx must be 0 (none), 1 (MX-fp8) or 2 (W4A8)")
    return m


# ----------------------------------------------------------------------------- stages


def router_logits(x, Wr, bias=None):
    x, Wr = _f32(x), _f32(Wr)
    T, H = x.shape
    E = Wr.shape[0]
    b = None if bias is None else _f32(bias)
    z = np.empty((T, E), np.float32)
    _check(_load().oracle_router_logits(T, H, E, _p(x), _p(Wr), _p(b), _p(z)), "router_logits")
    return z


def route(x, Wr, bias, k, rho, route_norm=True):
    """Gating.  Returns (topk_idx [T,k] int32, topk_w [T,k] fp32,
    scores [T,E] fp32, gap [T] fp32)."""
    x, Wr = _f32(x), _f32(Wr)
    T, H = x.shape
    E = Wr.shape[0]
    b = None if bias is None else _f32(bias)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    s = np.empty((T, E), np.float32)
    gap = np.empty((T,), np.float32)
    _check(_load().oracle_route(T, H, E, k, _p(x), _p(Wr), _p(b), ctypes.c_float(rho),
                                int(bool(route_norm)), _p(idx), _p(w), _p(s), _p(gap)), "route")
    return idx, w, s, gap


def route_weights(scores, topk_idx, rho, route_norm=True):
    """Gating step 4 on a given selection: topk_w [T,k] from this oracle's
    sigmoid scores [T,E] and the selected experts topk_idx [T,k] (k distinct
    experts per row)."""
    s = _f32(scores)
    idx = _i32(topk_idx)
    T, E = s.shape
    k = idx.shape[1]
    if idx.shape[0] != T:
        raise ValueError("scores and topk_idx disagree on T")
    w = np.empty((T, k), np.float32)
    _check(_load().oracle_route_weights(T, E, k, _p(s), _p(idx), ctypes.c_float(rho),
                                        int(bool(route_norm)), _p(w)), "route_weights")
    return w


def permute(topk_idx, E):
    """InitRouting.  Returns (counts [E], offsets [E+1], sorted_src [T*k], dest [T*k])."""
    idx = _i32(topk_idx)
    T, k = idx.shape
    counts = np.empty((E,), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    src = np.empty((T * k,), np.int32)
    dest = np.empty((T * k,), np.int32)
    _check(_load().oracle_permute(T, E, k, _p(idx), _p(counts), _p(offsets), _p(src), _p(dest)),
           "permute")
    return counts, offsets, src, dest


def swiglu_rows(xrows, Wg, Wu, Wd, mx=False):
    """One expert's SwiGLU FFN over rows.  Returns (h [M,I] pre-MX, y [M,H]).
    mx: 0/False none, 1/True MX-fp8 (W8A8), 2 W4A8 (MXFP4 weights)."""
    xrows = _f32(xrows)
    M, H = xrows.shape
    Wg, dt = _weights(Wg)
    Wu, dt2 = _weights(Wu)
    Wd, dt3 = _weights(Wd)
    if not (dt == dt2 == dt3):
        raise ValueError("mixed weight dtypes")
    I = Wg.shape[0]
    h = np.empty((M, I), np.float32)
    y = np.empty((M, H), np.float32)
    _check(_load().oracle_swiglu_rows(M, H, I, _p(xrows), dt, _p(Wg), _p(Wu), _p(Wd), _mx_mode(mx),
                                      _p(h), _p(y)), "swiglu_rows")
    return h, y


def combine(y, dest, topk_w, zsh=None):
    y = _f32(y)
    dest = _i32(dest)
    w = _f32(topk_w)
    T, k = w.shape
    H = y.shape[1]
    z = None if zsh is None else _f32(zsh)
    out = np.empty((T, H), np.float32)
    _check(_load().oracle_combine(T, H, k, _p(y), _p(dest), _p(w), _p(z), _p(out)), "combine")
    return out


def layer_forward(x, Wr, bias, Wg, Wu, Wd, Sg=None, Su=None, Sd=None, *, k, rho, route_norm=True,
                  mx=False):
    """The whole layer in the pages' order.  Weights: [E,I,H], [E,I,H], [E,H,I]
    (fp32 or bf16 bit patterns); shared [Is,H], [Is,H], [H,Is] or None.
    Returns a dict with out and every intermediate."""
    x, Wr = _f32(x), _f32(Wr)
    T, H = x.shape
    E = Wr.shape[0]
    Wg, dt = _weights(Wg)
    Wu, _ = _weights(Wu)
    Wd, _ = _weights(Wd)
    I = Wg.shape[1]
    if Sg is not None:
        Sg, _ = _weights(Sg)
        Su, _ = _weights(Su)
        Sd, _ = _weights(Sd)
        Is = Sg.shape[0]
    else:
        Is = 0
    b = None if bias is None else _f32(bias)
    P = T * k
    r = dict(out=np.empty((T, H), np.float32), topk_idx=np.empty((T, k), np.int32),
             topk_w=np.empty((T, k), np.float32), counts=np.empty((E,), np.int32),
             offsets=np.empty((E + 1,), np.int32), sorted_src=np.empty((P,), np.int32),
             dest=np.empty((P,), np.int32), h=np.empty((P, I), np.float32),
             y=np.empty((P, H), np.float32), zsh=np.zeros((T, H), np.float32))
    _check(_load().oracle_layer_forward(
        T, H, E, k, I, Is, ctypes.c_float(rho), int(bool(route_norm)), _p(x), _p(Wr), _p(b), dt,
        _p(Wg), _p(Wu), _p(Wd), _p(Sg), _p(Su), _p(Sd), _mx_mode(mx), _p(r["out"]),
        _p(r["topk_idx"]), _p(r["topk_w"]), _p(r["counts"]), _p(r["offsets"]),
        _p(r["sorted_src"]), _p(r["dest"]), _p(r["h"]), _p(r["y"]), _p(r["zsh"])),
        "layer_forward")
    return r


def layer_forward_tokens(tokens, x, Wr, bias, expert_weights, shared_weights, *, k, rho,
                         route_norm=True, mx=False, fp8=None, topk_idx=None):
    """Layer output for selected tokens only, straight from the definition.

    ``expert_weights(e)`` returns (Wg [I,H], Wu [I,H], Wd [H,I]) of expert e;
    ``shared_weights`` is (Sg, Su, Sd) or None.  ``fp8`` = (s_x, s_h, s_h_shared)
    selects static per-tensor FP8 experts (fp32 masters in, quantised here)
    with those activation scales; otherwise ``mx`` applies.  ``topk_idx``
    ([n,k], optional) replaces this oracle's selection for these tokens by a
    given one (whose weights then follow step 4 from this oracle's scores):
    how a token whose selection differs only by near-equal scores is
    evaluated.  Returns (out [n,H], topk_idx [n,k], topk_w [n,k], gap [n])
    for ``x[tokens]``."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = _f32(np.asarray(x)[tokens])
    idx, w, scores, gap = route(xs, Wr, bias, k, rho, route_norm)
    if topk_idx is not None:
        idx = _i32(topk_idx).reshape(len(tokens), k)
        w = route_weights(scores, idx, rho, route_norm)
    n, H = xs.shape
    out = np.empty((n, H), np.float32)
    # Evaluate each needed expert once over the tokens that picked it.
    rows_of = {}
    for i in range(n):
        for j in range(k):
            rows_of.setdefault(int(idx[i, j]), []).append((i, j))
    yk = np.empty((n, k, H), np.float32)
    for e, lst in sorted(rows_of.items()):
        Wg, Wu, Wd = expert_weights(e)
        rows = np.array([i for i, _ in lst])
        if fp8 is not None:
            _, y = swiglu_rows_fp8(xs[rows], Wg, Wu, Wd, fp8[0], fp8[1])
        else:
            _, y = swiglu_rows(xs[rows], Wg, Wu, Wd, mx=mx)
        for (i, j), yr in zip(lst, y):
            yk[i, j] = yr
    zsh = None
    if shared_weights is not None and fp8 is not None:
        _, zsh = swiglu_rows_fp8(xs, *shared_weights, fp8[0], fp8[2])
    elif shared_weights is not None:
        # the shared expert of a W4A8 layer stays W8A8
        _, zsh = swiglu_rows(xs, *shared_weights, mx=MX_FP8 if _mx_mode(mx) == MX_W4A8 else mx)
    # Rows of yk are already in (token, slot) order, so dest is the identity.
    dest = np.arange(n * k, dtype=np.int32)
    out = combine(yk.reshape(n * k, H), dest, w, zsh)
    return out, idx, w, gap
