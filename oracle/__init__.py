"""CPU oracle of the quantized linear layer (NumPy front end over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py import this package.  It shares no code with
the product library (weight_quantized_amd): it neither imports it nor is
imported by it.  Every function here is marshalling around the C routines
in oracle.c, whose header states the steps and the passages they follow.

Arrays are NumPy; fp16 tensors travel as uint16 bit patterns or float16.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = C.c_void_p
_i64 = C.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # built on first use when nothing is built yet
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    sig = {
        "or_f16_to_f32": (C.c_float, [C.c_uint16]),
        "or_f32_to_f16": (C.c_uint16, [C.c_float]),
        "or_f32_to_f16_up": (C.c_uint16, [C.c_float]),
        "or_f16_to_f32_n": (None, [_p, _i64, _p]),
        "or_f32_to_f16_n": (None, [_p, _i64, C.c_int, _p]),
        "or_awq_quantize": (C.c_int, [_p, _i64, _i64, C.c_int, _p, _p, _p]),
        "or_awq_pack": (C.c_int, [_p, _p, _i64, _i64, C.c_int, _p, _p]),
        "or_awq_unpack": (C.c_int, [_p, _p, _i64, _i64, C.c_int, _p, _p]),
        "or_awq_dequant": (C.c_int, [_p, _p, _p, _i64, _i64, C.c_int, _p, _p]),
        "or_w4a16_matmul": (C.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _p]),
        "or_w4a16_forward": (C.c_int, [_p, _i64, _p, _p, _p, _i64, _i64, C.c_int, _p, _i64, _p]),
        "or_sym_int4": (C.c_int, [_p, _i64, _p, _p]),
        "or_smooth": (C.c_int, [_p, _i64, _p, _p, _i64, _i64, _p, _p, _p]),
        "or_w8_quant_weight": (C.c_int, [_p, _i64, _i64, _p, _p]),
        "or_quant_rmsnorm": (C.c_int, [_p, _i64, _i64, _p, C.c_float, _p, _p, _p]),
        "or_int8_gemm": (C.c_int, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p]),
        "or_w8a8_forward": (C.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _p, _i64, _p, _i64, _p]),
        "or_add_quant_rmsnorm": (C.c_int, [_p, _p, _i64, _i64, _p, C.c_float, _p, _p, _p, _p]),
        "or_quant_per_token": (C.c_int, [_p, _i64, _i64, _p, _p]),
        "or_w8a8_forward_ex": (C.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _p, _i64, _p, _i64, _p]),
        "or_e4m3_to_f32": (C.c_float, [C.c_uint8]),
        "or_f32_to_e4m3": (C.c_uint8, [C.c_float]),
        "or_quant_fp8": (C.c_int, [_p, _i64, _i64, _p, C.c_float, _p, _p]),
        "or_fp8_quant_weight": (C.c_int, [_p, _i64, _i64, _p, _p]),
        "or_fp8_forward": (C.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _p, _i64, _p, _i64, _p]),
        "or_kv_quant_int8": (C.c_int, [_p, _i64, C.c_int, _p, _p]),
        "or_kv_dequant_int8": (C.c_int, [_p, _p, _i64, C.c_int, _p]),
        "or_f64_to_f16": (C.c_uint16, [C.c_double]),
        "or_awq_scales": (None, [_p, _p, _i64, C.c_double, _p]),
        "or_awq_search": (C.c_int, [_p, _i64, _p, _i64, _i64, C.c_int, C.c_int, C.c_int, _p, _p, _p]),
        "or_sumsq_exact": (None, [_p, _i64, _p, _p]),
        "or_ratio_to_f32_parts": (C.c_float, [C.c_uint64, C.c_uint64, C.c_uint64, C.c_int]),
        "or_num_threads": (C.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _bits16(a):
    a = np.asarray(a)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16)
    return _c(a, np.uint16)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


# ---------------------------------------------------------------- binary16
def f16_to_f32(h):
    """binary16 bit patterns (uint16 or float16 array) -> float32 values."""
    lib = _load()
    h = _bits16(h)
    out = np.empty(h.shape, np.float32)
    lib.or_f16_to_f32_n(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_f16(x):
    """float32 -> binary16 bit patterns (uint16), nearest, ties to even."""
    lib = _load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.or_f32_to_f16_n(_ptr(x), x.size, 0, _ptr(out))
    return out


def f32_to_f16_up(x):
    """float32 (finite, >= 2^-14) -> smallest binary16 >= x, as uint16 bits."""
    lib = _load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.or_f32_to_f16_n(_ptr(x), x.size, 1, _ptr(out))
    return out


# ---------------------------------------------------------------- W4A16
def awq_quantize(w, group):
    """Steps 1-4: returns (q uint8 [n,k], z uint8 [n,k/G], s fp16-bits uint16 [n,k/G])."""
    lib = _load()
    w = _c(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.uint8)
    z = np.empty((n, k // group), np.uint8)
    s = np.empty((n, k // group), np.uint16)
    _check(lib.or_awq_quantize(_ptr(w), n, k, group, _ptr(q), _ptr(z), _ptr(s)), "awq_quantize")
    return q, z, s


def awq_pack(q, z, group):
    """Step 5: returns (qweight int32 [n,k/8], qzeros int32 [n, ceil(k/G/8)])."""
    lib = _load()
    q = _c(q, np.uint8)
    z = _c(z, np.uint8)
    n, k = q.shape
    zw = (k // group + 7) // 8
    qw = np.empty((n, k // 8), np.uint32)
    qz = np.empty((n, zw), np.uint32)
    _check(lib.or_awq_pack(_ptr(q), _ptr(z), n, k, group, _ptr(qw), _ptr(qz)), "awq_pack")
    return qw.view(np.int32), qz.view(np.int32)


def awq_unpack(qweight, qzeros, group):
    """Step 6: returns (q uint8 [n,k], z uint8 [n,k/G])."""
    lib = _load()
    qw = _c(np.asarray(qweight).view(np.uint32), np.uint32)
    qz = _c(np.asarray(qzeros).view(np.uint32), np.uint32)
    n, k8 = qw.shape
    k = k8 * 8
    q = np.empty((n, k), np.uint8)
    z = np.empty((n, k // group), np.uint8)
    _check(lib.or_awq_unpack(_ptr(qw), _ptr(qz), n, k, group, _ptr(q), _ptr(z)), "awq_unpack")
    return q, z


def awq_dequant(q, z, s, group):
    """Step 7: returns (wd float32 [n,k], wd16 float16 [n,k])."""
    lib = _load()
    q = _c(q, np.uint8)
    z = _c(z, np.uint8)
    s = _bits16(s)
    n, k = q.shape
    wd = np.empty((n, k), np.float32)
    wd16 = np.empty((n, k), np.uint16)
    _check(lib.or_awq_dequant(_ptr(q), _ptr(z), _ptr(s), n, k, group, _ptr(wd), _ptr(wd16)), "awq_dequant")
    return wd, wd16.view(np.float16)


def w4a16_matmul(x, wd16, rows=None):
    """Step 8: y float64 [m, len(rows) or n] = x @ wd16[rows].T with an fp64 accumulator."""
    lib = _load()
    x = _bits16(x)
    w = _bits16(wd16)
    m, k = x.shape
    n = w.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = n if r is None else len(r)
    y = np.empty((m, nr), np.float64)
    _check(lib.or_w4a16_matmul(_ptr(x), m, _ptr(w), n, k, _ptr(r), nr, _ptr(y)), "w4a16_matmul")
    return y


def w4a16_forward(x, qweight, scales, qzeros, group, rows=None):
    """Steps 6-8 from packed tensors for output channels `rows` (all if None)."""
    lib = _load()
    x = _bits16(x)
    qw = _c(np.asarray(qweight).view(np.uint32), np.uint32)
    qz = _c(np.asarray(qzeros).view(np.uint32), np.uint32)
    s = _bits16(scales)
    m, k = x.shape
    n = qw.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = n if r is None else len(r)
    y = np.empty((m, nr), np.float64)
    _check(lib.or_w4a16_forward(_ptr(x), m, _ptr(qw), _ptr(s), _ptr(qz), n, k, group, _ptr(r), nr, _ptr(y)),
           "w4a16_forward")
    return y


def sym_int4(w):
    """Symmetric per-tensor int4 of the worked example: (scale, q int8)."""
    lib = _load()
    w = _c(w, np.float32)
    q = np.empty(w.shape, np.int8)
    sc = np.zeros(1, np.float32)
    lib.or_sym_int4(_ptr(w), w.size, _ptr(sc), _ptr(q))
    return np.float32(sc[0]), q


# ---------------------------------------------------------------- W8A8
def smooth(x, gamma, w):
    """Steps 1-2: (s float32 [k], gamma' float16 [k], W' float32 [n,k])."""
    lib = _load()
    x = _bits16(x)
    g = _bits16(gamma)
    w = _c(w, np.float32)
    rows, k = x.shape
    n = w.shape[0]
    s = np.empty(k, np.float32)
    gs = np.empty(k, np.uint16)
    ws = np.empty((n, k), np.float32)
    _check(lib.or_smooth(_ptr(x), rows, _ptr(g), _ptr(w), n, k, _ptr(s), _ptr(gs), _ptr(ws)), "smooth")
    return s, gs.view(np.float16), ws


def w8_quant_weight(w):
    """Step 3: (wq int8 [n,k], w_scale float32 [n])."""
    lib = _load()
    w = _c(w, np.float32)
    n, k = w.shape
    wq = np.empty((n, k), np.int8)
    sc = np.empty(n, np.float32)
    lib.or_w8_quant_weight(_ptr(w), n, k, _ptr(wq), _ptr(sc))
    return wq, sc


def quant_rmsnorm(x, gamma, eps=1e-6, return_ms=False):
    """Step 4: (xq int8 [m,k], x_scale float32 [m]) [, ms float32 [m]]."""
    lib = _load()
    x = _bits16(x)
    g = _bits16(gamma)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    sc = np.empty(m, np.float32)
    ms = np.empty(m, np.float32)
    _check(lib.or_quant_rmsnorm(_ptr(x), m, k, _ptr(g), float(eps), _ptr(xq), _ptr(sc), _ptr(ms)),
           "quant_rmsnorm")
    return (xq, sc, ms) if return_ms else (xq, sc)


def add_quant_rmsnorm(x, residual, gamma, eps=1e-6):
    """Step 7: (h fp16 bits uint16 [m,k], xq int8 [m,k], x_scale float32 [m])."""
    lib = _load()
    x = _bits16(x)
    r = _bits16(residual)
    g = _bits16(gamma)
    m, k = x.shape
    if r.shape != (m, k):
        raise ValueError("residual shape differs from x")
    h = np.empty((m, k), np.uint16)
    xq = np.empty((m, k), np.int8)
    sc = np.empty(m, np.float32)
    _check(lib.or_add_quant_rmsnorm(_ptr(x), _ptr(r), m, k, _ptr(g), float(eps), _ptr(h), _ptr(xq), _ptr(sc),
                                    None), "add_quant_rmsnorm")
    return h, xq, sc


def quant_per_token(x):
    """Step 8: (xq int8 [m,k], x_scale float32 [m])."""
    lib = _load()
    x = _bits16(x)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    sc = np.empty(m, np.float32)
    _check(lib.or_quant_per_token(_ptr(x), m, k, _ptr(xq), _ptr(sc)), "quant_per_token")
    return xq, sc


def int8_gemm(xq, wq, rows=None, cols=None):
    """Step 5: exact int64 acc [rows, cols] = xq[rows] @ wq[cols].T."""
    lib = _load()
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    m, k = xq.shape
    n = wq.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = m if r is None else len(r)
    nc = n if c is None else len(c)
    acc = np.empty((nr, nc), np.int64)
    lib.or_int8_gemm(_ptr(xq), m, _ptr(wq), n, k, _ptr(r), nr, _ptr(c), nc, _ptr(acc))
    return acc


def w8a8_forward(xq, x_scale, wq, w_scale, rows=None, cols=None):
    """Steps 5-6: y float64 [rows, cols]."""
    lib = _load()
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    xs = _c(x_scale, np.float32)
    ws = _c(w_scale, np.float32)
    m, k = xq.shape
    n = wq.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = m if r is None else len(r)
    nc = n if c is None else len(c)
    y = np.empty((nr, nc), np.float64)
    _check(lib.or_w8a8_forward(_ptr(xq), _ptr(xs), m, _ptr(wq), _ptr(ws), n, k, _ptr(r), nr, _ptr(c), nc,
                               _ptr(y)), "w8a8_forward")
    return y


def w8a8_forward_ex(xq, x_scale, wq, w_scale, bias=None, residual=None, rows=None, cols=None):
    """Step 9: y float64 [rows, cols] = acc * x_scale * w_scale + bias + residual
    (bias fp16 [n], residual fp16 [m, n], either None)."""
    lib = _load()
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    xs = _c(x_scale, np.float32)
    ws = _c(w_scale, np.float32)
    m, k = xq.shape
    n = wq.shape[0]
    b = None if bias is None else _bits16(bias)
    res = None if residual is None else _bits16(residual)
    if b is not None and b.shape != (n,):
        raise ValueError("bias must be [n]")
    if res is not None and res.shape != (m, n):
        raise ValueError("residual must be [m, n]")
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = m if r is None else len(r)
    nc = n if c is None else len(c)
    y = np.empty((nr, nc), np.float64)
    _check(lib.or_w8a8_forward_ex(_ptr(xq), _ptr(xs), m, _ptr(wq), _ptr(ws), n, k, _ptr(b), _ptr(res), _ptr(r), nr,
                                  _ptr(c), nc, _ptr(y)), "w8a8_forward_ex")
    return y


# ---------------------------------------------------------------- FP8 E4M3
def e4m3_to_f32(codes):
    """e4m3 bytes (uint8 array) -> float32 values (NaN for the NaN codes)."""
    lib = _load()
    c = _c(codes, np.uint8)
    return np.array([lib.or_e4m3_to_f32(int(v)) for v in c.ravel()], np.float32).reshape(c.shape)


def f32_to_e4m3(x):
    """float32 -> e4m3 bytes, nearest with ties to even (NaN above 464)."""
    lib = _load()
    x = _c(x, np.float32)
    return np.array([lib.or_f32_to_e4m3(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def quant_fp8(x, gamma=None, eps=1e-6):
    """Step 10 on activations: (xq e4m3 bytes [m,k], x_scale float32 [m]);
    RMSNorm first when gamma is given, else the plain per-token cast."""
    lib = _load()
    x = _bits16(x)
    g = None if gamma is None else _bits16(gamma)
    m, k = x.shape
    xq = np.empty((m, k), np.uint8)
    sc = np.empty(m, np.float32)
    _check(lib.or_quant_fp8(_ptr(x), m, k, _ptr(g), float(eps), _ptr(xq), _ptr(sc)), "quant_fp8")
    return xq, sc


def fp8_quant_weight(w):
    """Step 10 on weights: (wq e4m3 bytes [n,k], w_scale float32 [n])."""
    lib = _load()
    w = _c(w, np.float32)
    n, k = w.shape
    wq = np.empty((n, k), np.uint8)
    sc = np.empty(n, np.float32)
    _check(lib.or_fp8_quant_weight(_ptr(w), n, k, _ptr(wq), _ptr(sc)), "fp8_quant_weight")
    return wq, sc


def fp8_forward(xq, x_scale, wq, w_scale, rows=None, cols=None):
    """Step 11: y float64 [rows, cols]; the bare accumulator when the scales are None."""
    lib = _load()
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    xs = None if x_scale is None else _c(x_scale, np.float32)
    ws = None if w_scale is None else _c(w_scale, np.float32)
    m, k = xq.shape
    n = wq.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = m if r is None else len(r)
    nc = n if c is None else len(c)
    y = np.empty((nr, nc), np.float64)
    _check(lib.or_fp8_forward(_ptr(xq), _ptr(xs), m, _ptr(wq), _ptr(ws), n, k, _ptr(r), nr, _ptr(c), nc, _ptr(y)),
           "fp8_forward")
    return y


# ---------------------------------------------------------------- KV cache INT8
def kv_quant_int8(x, group=128):
    """Step 12: x fp16 [..., G-multiple] -> (q int8 same shape, scale float32 [groups])."""
    lib = _load()
    xb = _bits16(x)
    if xb.size % group:
        raise ValueError("size must be a multiple of the group")
    groups = xb.size // group
    q = np.empty(xb.shape, np.int8)
    sc = np.empty(groups, np.float32)
    _check(lib.or_kv_quant_int8(_ptr(xb), groups, int(group), _ptr(q), _ptr(sc)), "kv_quant_int8")
    return q, sc


def kv_dequant_int8(q, scale, group=128):
    """Step 12, dequantisation: fp16 bits (uint16) of q * scale, q's shape."""
    lib = _load()
    q = _c(q, np.int8)
    sc = _c(scale, np.float32)
    groups = q.size // group
    if q.size % group or sc.size != groups:
        raise ValueError("q and scale do not match the group")
    out = np.empty(q.shape, np.uint16)
    _check(lib.or_kv_dequant_int8(_ptr(q), _ptr(sc), groups, int(group), _ptr(out)), "kv_dequant_int8")
    return out


# ---------------------------------------------------------------- AWQ scale search
def f64_to_f16(v):
    """binary16 bits of a float64 value, rounded once to nearest even."""
    return int(_load().or_f64_to_f16(float(v)))


def awq_scales(a, b, alpha):
    """Step 14's smoothing vector s float32 [k] from the column maxima a, b."""
    lib = _load()
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    s = np.empty(a.size, np.float32)
    lib.or_awq_scales(_ptr(a), _ptr(b), a.size, float(alpha), _ptr(s))
    return s


def awq_search(x, w, group, grid=20, quant=True):
    """Steps 13-15: (err float64 [grid], best int, s_best float32 [k]) for
    calibration tokens x (fp16 [t, k]) and weights w (float32 [n, k])."""
    lib = _load()
    x = _bits16(x)
    w = _c(w, np.float32)
    t, k = x.shape
    n = w.shape[0]
    err = np.empty(int(grid), np.float64)
    best = np.zeros(1, np.int32)
    s = np.empty(k, np.float32)
    _check(lib.or_awq_search(_ptr(x), t, _ptr(w), n, k, int(group), int(grid), int(bool(quant)), _ptr(err),
                             _ptr(best), _ptr(s)), "awq_search")
    return err, int(best[0]), s


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().or_num_threads())


def sumsq_exact(x_row):
    """Exact sum of squares of an fp16 row, as a Python int in units of 2^-48."""
    lib = _load()
    x = _bits16(x_row)
    hi = C.c_uint64()
    lo = C.c_uint64()
    lib.or_sumsq_exact(_ptr(x), x.size, C.byref(hi), C.byref(lo))
    return (hi.value << 64) | lo.value


def ratio_to_f32(num: int, den: int, e2: int) -> np.float32:
    """num / den * 2**e2 rounded to the nearest float32 (ties to even)."""
    lib = _load()
    return np.float32(lib.or_ratio_to_f32_parts(num >> 64, num & ((1 << 64) - 1), den, e2))
