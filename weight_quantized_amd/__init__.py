"""Python binding of libqlinear, the MI355X quantized linear layer.

Argument marshalling only: every step runs in libqlinear (HIP kernels for
gfx950 and the host quantisers).  Device tensors are torch tensors on the
current HIP device; PyTorch supplies memory and the current stream.  Host
functions take and return NumPy arrays.

The library must have been built (``python -m weight_quantized_amd.build``);
importing the package without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

__all__ = [
    "QLError", "lib_path", "awq_pack", "smooth", "w8a8_quant_weight",
    "w4a16_workspace_bytes", "w4a16_gemm", "w4a16_dequant", "w8a8_quant_rmsnorm",
    "w8a8_gemm", "w8a8_gemm_i32", "status_string", "version",
    "PATH_AUTO", "PATH_DECODE", "PATH_GEMM", "W4A16_WS_ZERO_BYTES", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libqlinear.so")

PATH_AUTO, PATH_DECODE, PATH_GEMM = 0, 1, 2

# Leading bytes of a W4A16 workspace that are zero between calls (split-K
# arrival counters, then two-slice exchange slots); mirrors include/qlinear.h
W4A16_WS_ZERO_BYTES = 32768 + (4 << 20)

_p, _i64, _sz, _i = C.c_void_p, C.c_int64, C.c_size_t, C.c_int

# name -> (restype, argtypes); mirrors include/qlinear.h
EXPORTS = {
    "ql_awq_pack": (_i, [_p, _i64, _i64, _i, _p, _p, _p]),
    "ql_awq_search_workspace_bytes": (_sz, [_i64, _i64, _i64, _i]),
    "ql_awq_search": (_i, [_p, _i64, _p, _i64, _i64, _i, _i, _p, _sz, _p, _p, _p, _p, _p, _p, _p]),
    "ql_w4a16_workspace_bytes": (_sz, [_i64, _i64, _i64, _i]),
    "ql_w4a16_gemm": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i, _p, _sz, _p]),
    "ql_w4a16_gemm_path": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i, _p, _sz, _p, _i]),
    "ql_w4a16_gemm_noalloc": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i, _p]),
    "ql_w4a16_dequant": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i, _p]),
    "ql_smooth": (_i, [_p, _i64, _p, _p, _i64, _i64, _p, _p, _p]),
    "ql_w8a8_quant_weight": (_i, [_p, _i64, _i64, _p, _p]),
    "ql_w8a8_quant_rmsnorm": (_i, [_p, _p, C.c_float, _p, _p, _i64, _i64, _p]),
    "ql_w8a8_gemm": (_i, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "ql_w8a8_add_quant_rmsnorm": (_i, [_p, _p, _p, C.c_float, _p, _p, _p, _i64, _i64, _p]),
    "ql_w8a8_quant_per_token": (_i, [_p, _p, _p, _i64, _i64, _p]),
    "ql_w8a8_gemm_ex": (_i, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "ql_w8a8_gemm_i32": (_i, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "ql_kv_quant_int8": (_i, [_p, _p, _p, _i64, _i, _p]),
    "ql_kv_dequant_int8": (_i, [_p, _p, _p, _i64, _i, _p]),
    "ql_fp8_quant_weight": (_i, [_p, _i64, _i64, _p, _p]),
    "ql_fp8_quant_rmsnorm": (_i, [_p, _p, C.c_float, _p, _p, _i64, _i64, _p]),
    "ql_fp8_quant_per_token": (_i, [_p, _p, _p, _i64, _i64, _p]),
    "ql_fp8_gemm": (_i, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "ql_status_string": (C.c_char_p, [_i]),
    "ql_last_error": (C.c_char_p, []),
    "ql_version": (_i, []),
}

if not os.path.exists(lib_path):
    raise ImportError(f"libqlinear.so not built at {lib_path}; run `python -m weight_quantized_amd.build`")

# torch first: its HIP runtime (libamdhip64.so.7) is then already loaded and the
# library binds to that one instance instead of mapping a second runtime.
import torch  # noqa: E402,F401

_lib = C.CDLL(lib_path)
for _name, (_res, _args) in EXPORTS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class QLError(RuntimeError):
    """A libqlinear call returned a QL_ERR_* status."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{status_string(code)} ({code}): {msg}")
        self.code = code


def status_string(code: int) -> str:
    return _lib.ql_status_string(code).decode()


def version() -> int:
    return _lib.ql_version()


def _check(rc: int):
    if rc != 0:
        raise QLError(rc, _lib.ql_last_error().decode())


def _np(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _f16_bits(a):
    a = np.asarray(a)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a)
    raise TypeError(f"expected float16, got {a.dtype}")


# ---------------------------------------------------------------- host
def awq_pack(w, group: int):
    """float32 w [n, k] -> (qweight int32 [n, k/8], scales float16 [n, k/group],
    qzeros int32 [n, ceil(k/group/8)])."""
    w = _np(w, np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    n, k = w.shape
    g = max(int(group), 1)
    qw = np.empty((n, k // 8), np.int32)
    sc = np.empty((n, k // g), np.uint16)
    qz = np.empty((n, (k // g + 7) // 8), np.int32)
    _check(_lib.ql_awq_pack(w.ctypes.data, n, k, int(group), qw.ctypes.data, sc.ctypes.data, qz.ctypes.data))
    return qw, sc.view(np.float16), qz


def awq_search(x, w, group: int, grid: int = 20, device=None):
    """AWQ ratio search over calibration tokens x (fp16 [t, k], host) for
    weights w (float32 [n, k], host), each candidate scored with the device
    GEMM.  Returns (err float64 [grid], best int, s float32 [k],
    (qweight, scales, qzeros) of the chosen smoothed weights)."""
    torch = _torch()
    x = _f16_bits(x)
    w = _np(w, np.float32)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x [t, k] and w [n, k] must share k")
    t, k = x.shape
    n = w.shape[0]
    g = max(int(group), 1)
    dev = torch.device("cuda:0") if device is None else torch.device(device)
    need = awq_search_workspace_bytes(t, n, k, group)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    err = np.empty(max(int(grid), 1), np.float64)
    best = np.zeros(1, np.int32)
    s = np.empty(k, np.float32)
    qw = np.empty((n, k // 8), np.int32)
    sc = np.empty((n, k // g), np.uint16)
    qz = np.empty((n, (k // g + 7) // 8), np.int32)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _check(_lib.ql_awq_search(x.ctypes.data, t, w.ctypes.data, n, k, int(group), int(grid), ws.data_ptr(),
                                  ws.numel(), stream, err.ctypes.data, best.ctypes.data, s.ctypes.data,
                                  qw.ctypes.data, sc.ctypes.data, qz.ctypes.data))
    return err[:int(grid)], int(best[0]), s, (qw, sc.view(np.float16), qz)


def awq_search_workspace_bytes(t: int, n: int, k: int, group: int) -> int:
    return int(_lib.ql_awq_search_workspace_bytes(t, n, k, int(group)))


def smooth(x, gamma, w):
    """SmoothQuant smoothing (alpha = 0.5): (s float32 [k], gamma' float16 [k], W' float32 [n, k])."""
    x = _f16_bits(x)
    gm = _f16_bits(gamma)
    w = _np(w, np.float32)
    rows, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k or gm.shape != (k,):
        raise ValueError("shape mismatch")
    s = np.empty(k, np.float32)
    gs = np.empty(k, np.uint16)
    ws = np.empty((n, k), np.float32)
    _check(_lib.ql_smooth(x.ctypes.data, rows, gm.ctypes.data, w.ctypes.data, n, k,
                          s.ctypes.data, gs.ctypes.data, ws.ctypes.data))
    return s, gs.view(np.float16), ws


def w8a8_quant_weight(w):
    """Per-channel symmetric int8: (wq int8 [n, k], w_scale float32 [n])."""
    w = _np(w, np.float32)
    n, k = w.shape
    wq = np.empty((n, k), np.int8)
    sc = np.empty(n, np.float32)
    _check(_lib.ql_w8a8_quant_weight(w.ctypes.data, n, k, wq.ctypes.data, sc.ctypes.data))
    return wq, sc


# ---------------------------------------------------------------- device
def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _shape(t, shape, name):
    """Raise ValueError unless tensor t has exactly `shape`."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _same_device(ref, *ts):
    for name, t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _mat(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t


def _out(out, shape, dtype, like, name="out"):
    """A caller-supplied output checked against (shape, dtype, device), or a
    new one."""
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _dev(out, dtype, name)
    _shape(out, shape, name)
    _same_device(like, (name, out))
    return out


def _w4_operands(qweight, scales, qzeros, n, k, group):
    """Check the packed-weight tensors of an [n, k] layer against the layout
    ql_awq_pack writes."""
    g = int(group)
    if g not in (32, 64, 128):
        raise ValueError(f"group {g} not in (32, 64, 128)")
    if k % g:
        raise ValueError(f"k={k} is not a multiple of the group {g}")
    _shape(qweight, (n, k // 8), "qweight")
    _shape(scales, (n, k // g), "scales")
    _shape(qzeros, (n, (k // g + 7) // 8), "qzeros")


def w4a16_workspace_bytes(m: int, n: int, k: int, group: int) -> int:
    return int(_lib.ql_w4a16_workspace_bytes(m, n, k, group))


_workspaces = {}


def _workspace(device, nbytes):
    """A zero-filled split-K workspace per (device, stream), grown on demand.
    The kernels leave its leading W4A16_WS_ZERO_BYTES (counters and exchange
    slots) zero after every call, so it is reused as is.  Calls on one stream run in order and may share it; calls on
    different streams may run concurrently and so each stream has its own.
    It is allocated while its stream is current, so when a larger one
    replaces it the caching allocator hands the old memory out again only to
    work ordered after the kernels already queued on that stream.  Under
    graph capture nothing is allocated: pass `workspace` explicitly there."""
    torch = _torch()
    if torch.cuda.is_current_stream_capturing():
        raise ValueError("w4a16_gemm under graph capture needs an explicit zero-filled workspace "
                         f"of at least {nbytes} bytes")
    stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def w4a16_gemm(x, qweight, scales, qzeros, group: int, out=None, workspace=None, path: int = PATH_AUTO):
    """y fp16 [m, n] = x fp16 [m, k] @ dequant(W)^T."""
    torch = _torch()
    x = _dev(x, torch.float16, "x")
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float16, "scales")
    qzeros = _dev(qzeros, torch.int32, "qzeros")
    m, k = _mat(x, "x").shape
    n = _mat(qweight, "qweight").shape[0]
    _w4_operands(qweight, scales, qzeros, n, k, group)
    _same_device(x, ("qweight", qweight), ("scales", scales), ("qzeros", qzeros))
    out = _out(out, (m, n), torch.float16, x)
    need = w4a16_workspace_bytes(m, n, k, group)
    if workspace is None:
        workspace = _workspace(x.device, need) if need else None
    else:
        _dev(workspace, torch.uint8, "workspace")
        _same_device(x, ("workspace", workspace))
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.ql_w4a16_gemm_path(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(),
                                   out.data_ptr(), m, n, k, int(group), wptr, wbytes, _stream(x), int(path)))
    return out


def w4a16_gemm_noalloc(x, qweight, scales, qzeros, group: int, out):
    """y fp16 [m, n] = x fp16 [m, k] @ dequant(W)^T into the caller's `out`,
    with the split-K scratch held by the library (nothing is allocated)."""
    torch = _torch()
    x = _dev(x, torch.float16, "x")
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float16, "scales")
    qzeros = _dev(qzeros, torch.int32, "qzeros")
    m, k = _mat(x, "x").shape
    n = _mat(qweight, "qweight").shape[0]
    _w4_operands(qweight, scales, qzeros, n, k, group)
    _same_device(x, ("qweight", qweight), ("scales", scales), ("qzeros", qzeros))
    if out is None:
        raise ValueError("w4a16_gemm_noalloc writes into a caller-supplied `out`")
    out = _out(out, (m, n), torch.float16, x)
    _check(_lib.ql_w4a16_gemm_noalloc(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(),
                                      out.data_ptr(), m, n, k, int(group), _stream(x)))
    return out


def w4a16_dequant(qweight, scales, qzeros, group: int, with_codes: bool = False):
    """Dequantised fp16 weights [n, k] (and uint8 codes [n, k] if with_codes)."""
    torch = _torch()
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float16, "scales")
    qzeros = _dev(qzeros, torch.int32, "qzeros")
    n, k = _mat(qweight, "qweight").shape[0], qweight.shape[1] * 8
    _w4_operands(qweight, scales, qzeros, n, k, group)
    _same_device(qweight, ("scales", scales), ("qzeros", qzeros))
    w16 = torch.empty((n, k), dtype=torch.float16, device=qweight.device)
    q8 = torch.empty((n, k), dtype=torch.uint8, device=qweight.device) if with_codes else None
    _check(_lib.ql_w4a16_dequant(qweight.data_ptr(), scales.data_ptr(), qzeros.data_ptr(), w16.data_ptr(),
                                 q8.data_ptr() if q8 is not None else None, n, k, int(group), _stream(qweight)))
    return (w16, q8) if with_codes else w16


def _token_outputs(x, xq, x_scale, code_dtype):
    torch = _torch()
    m, k = x.shape
    return (_out(xq, (m, k), code_dtype, x, "xq"), _out(x_scale, (m,), torch.float32, x, "x_scale"))


def _gamma(gamma, x):
    torch = _torch()
    gamma = _dev(gamma, torch.float16, "gamma")
    _shape(gamma, (x.shape[1],), "gamma")
    _same_device(x, ("gamma", gamma))
    return gamma


def w8a8_quant_rmsnorm(x, gamma, eps: float = 1e-6, xq=None, x_scale=None):
    """QRMSNorm: (xq int8 [m, k], x_scale float32 [m])."""
    torch = _torch()
    x = _mat(_dev(x, torch.float16, "x"), "x")
    gamma = _gamma(gamma, x)
    m, k = x.shape
    xq, x_scale = _token_outputs(x, xq, x_scale, torch.int8)
    _check(_lib.ql_w8a8_quant_rmsnorm(x.data_ptr(), gamma.data_ptr(), float(eps), xq.data_ptr(),
                                      x_scale.data_ptr(), m, k, _stream(x)))
    return xq, x_scale


def w8a8_add_quant_rmsnorm(x, residual, gamma, eps: float = 1e-6, h_out=None, xq=None, x_scale=None):
    """Residual-fused QRMSNorm: h = fp16(x + residual) is written to h_out
    (pass h_out=residual, or x, to update in place), then QRMSNorm of h.
    Returns (h, xq int8 [m, k], x_scale float32 [m])."""
    torch = _torch()
    x = _mat(_dev(x, torch.float16, "x"), "x")
    residual = _dev(residual, torch.float16, "residual")
    _shape(residual, x.shape, "residual")
    _same_device(x, ("residual", residual))
    gamma = _gamma(gamma, x)
    m, k = x.shape
    h_out = _out(h_out, (m, k), torch.float16, x, "h_out")
    xq, x_scale = _token_outputs(x, xq, x_scale, torch.int8)
    _check(_lib.ql_w8a8_add_quant_rmsnorm(x.data_ptr(), residual.data_ptr(), gamma.data_ptr(), float(eps),
                                          h_out.data_ptr(), xq.data_ptr(), x_scale.data_ptr(), m, k, _stream(x)))
    return h_out, xq, x_scale


def w8a8_quant_per_token(x, xq=None, x_scale=None):
    """Per-token int8 quantisation of a plain activation: (xq int8 [m, k],
    x_scale float32 [m]) with x_scale = max|x| / 127."""
    torch = _torch()
    x = _mat(_dev(x, torch.float16, "x"), "x")
    m, k = x.shape
    xq, x_scale = _token_outputs(x, xq, x_scale, torch.int8)
    _check(_lib.ql_w8a8_quant_per_token(x.data_ptr(), xq.data_ptr(), x_scale.data_ptr(), m, k, _stream(x)))
    return xq, x_scale


def _gemm8_operands(xq, x_scale, wq, w_scale, code_dtype):
    """Check the 8-bit GEMM operands: xq [m, k], x_scale [m], wq [n, k],
    w_scale [n], all on one device; returns (m, n, k)."""
    torch = _torch()
    _dev(xq, code_dtype, "xq")
    _dev(wq, code_dtype, "wq")
    m, k = _mat(xq, "xq").shape
    n = _mat(wq, "wq").shape[0]
    _shape(wq, (n, k), "wq")
    _same_device(xq, ("wq", wq))
    if x_scale is not None:
        _dev(x_scale, torch.float32, "x_scale")
        _shape(x_scale, (m,), "x_scale")
        _dev(w_scale, torch.float32, "w_scale")
        _shape(w_scale, (n,), "w_scale")
        _same_device(xq, ("x_scale", x_scale), ("w_scale", w_scale))
    return m, n, k


def _epilogue_terms(bias, residual, m, n, like):
    torch = _torch()
    if bias is not None:
        bias = _dev(bias, torch.float16, "bias")
        _shape(bias, (n,), "bias")
    if residual is not None:
        residual = _dev(residual, torch.float16, "residual")
        _shape(residual, (m, n), "residual")
    _same_device(like, ("bias", bias), ("residual", residual))
    return bias, residual


def w8a8_gemm_ex(xq, x_scale, wq, w_scale, bias=None, residual=None, out=None):
    """y fp16 [m, n] = fp16((xq @ wq^T) * x_scale * w_scale [+ bias] [+ residual]),
    bias fp16 [n], residual fp16 [m, n]; out may be residual (in place)."""
    torch = _torch()
    m, n, k = _gemm8_operands(xq, x_scale, wq, w_scale, torch.int8)
    bias, residual = _epilogue_terms(bias, residual, m, n, xq)
    out = _out(out, (m, n), torch.float16, xq)
    _check(_lib.ql_w8a8_gemm_ex(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(),
                                bias.data_ptr() if bias is not None else None,
                                residual.data_ptr() if residual is not None else None, out.data_ptr(), m, n, k,
                                _stream(xq)))
    return out


def w8a8_gemm(xq, x_scale, wq, w_scale, out=None):
    """y fp16 [m, n] = fp16((xq @ wq^T) * x_scale[:, None] * w_scale[None, :])."""
    torch = _torch()
    m, n, k = _gemm8_operands(xq, x_scale, wq, w_scale, torch.int8)
    out = _out(out, (m, n), torch.float16, xq)
    _check(_lib.ql_w8a8_gemm(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(),
                             out.data_ptr(), m, n, k, _stream(xq)))
    return out


def fp8_quant_weight(w):
    """Per-channel FP8 E4M3 weights: (wq uint8 codes [n, k], w_scale float32 [n])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    wq = np.empty((n, k), np.uint8)
    sc = np.empty(n, np.float32)
    _check(_lib.ql_fp8_quant_weight(w.ctypes.data, n, k, wq.ctypes.data, sc.ctypes.data))
    return wq, sc


def fp8_quant_rmsnorm(x, gamma, eps: float = 1e-6, xq=None, x_scale=None):
    """QRMSNorm with FP8 E4M3 codes: (xq uint8 [m, k], x_scale float32 [m])."""
    torch = _torch()
    x = _mat(_dev(x, torch.float16, "x"), "x")
    gamma = _gamma(gamma, x)
    m, k = x.shape
    xq, x_scale = _token_outputs(x, xq, x_scale, torch.uint8)
    _check(_lib.ql_fp8_quant_rmsnorm(x.data_ptr(), gamma.data_ptr(), float(eps), xq.data_ptr(),
                                     x_scale.data_ptr(), m, k, _stream(x)))
    return xq, x_scale


def fp8_quant_per_token(x, xq=None, x_scale=None):
    """Per-token FP8 E4M3 quantisation: (xq uint8 [m, k], x_scale float32 [m])."""
    torch = _torch()
    x = _mat(_dev(x, torch.float16, "x"), "x")
    m, k = x.shape
    xq, x_scale = _token_outputs(x, xq, x_scale, torch.uint8)
    _check(_lib.ql_fp8_quant_per_token(x.data_ptr(), xq.data_ptr(), x_scale.data_ptr(), m, k, _stream(x)))
    return xq, x_scale


def fp8_gemm(xq, x_scale, wq, w_scale, bias=None, residual=None, out=None):
    """y fp16 [m, n] = fp16(sum(e4m3 xq * e4m3 wq) * x_scale * w_scale [+ bias] [+ residual])."""
    torch = _torch()
    m, n, k = _gemm8_operands(xq, x_scale, wq, w_scale, torch.uint8)
    bias, residual = _epilogue_terms(bias, residual, m, n, xq)
    out = _out(out, (m, n), torch.float16, xq)
    _check(_lib.ql_fp8_gemm(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(),
                            bias.data_ptr() if bias is not None else None,
                            residual.data_ptr() if residual is not None else None, out.data_ptr(), m, n, k,
                            _stream(xq)))
    return out


def kv_quant_int8(x, group: int = 128, q=None, scale=None):
    """KV-cache INT8 groups: (q int8, x's shape; scale float32 [x.numel() // group])."""
    torch = _torch()
    x = _dev(x, torch.float16, "x")
    if int(group) not in (32, 64, 128):
        raise ValueError(f"group {group} not in (32, 64, 128)")
    if x.numel() % group:
        raise ValueError("x's size must be a multiple of the group")
    groups = x.numel() // group
    q = _out(q, tuple(x.shape), torch.int8, x, "q")
    scale = _out(scale, (groups,), torch.float32, x, "scale")
    _check(_lib.ql_kv_quant_int8(x.data_ptr(), q.data_ptr(), scale.data_ptr(), groups, int(group), _stream(x)))
    return q, scale


def kv_dequant_int8(q, scale, group: int = 128, out=None):
    """fp16 values of KV-cache INT8 groups, q's shape."""
    torch = _torch()
    q = _dev(q, torch.int8, "q")
    scale = _dev(scale, torch.float32, "scale")
    if int(group) not in (32, 64, 128):
        raise ValueError(f"group {group} not in (32, 64, 128)")
    if q.numel() % group:
        raise ValueError("q's size must be a multiple of the group")
    _shape(scale, (q.numel() // group,), "scale")
    _same_device(q, ("scale", scale))
    out = _out(out, tuple(q.shape), torch.float16, q)
    _check(_lib.ql_kv_dequant_int8(q.data_ptr(), scale.data_ptr(), out.data_ptr(), q.numel() // group, int(group),
                                   _stream(q)))
    return out


def w8a8_gemm_i32(xq, wq, out=None):
    """Raw int32 accumulator [m, n] = xq @ wq^T."""
    torch = _torch()
    m, n, k = _gemm8_operands(xq, None, wq, None, torch.int8)
    out = _out(out, (m, n), torch.int32, xq)
    _check(_lib.ql_w8a8_gemm_i32(xq.data_ptr(), wq.data_ptr(), out.data_ptr(), m, n, k, _stream(xq)))
    return out
