"""The C ABI: library loads, exports every symbol of include/qlinear.h, and
rejects bad arguments with the documented codes before launching anything.

CPU only.  Every device-side call here fails validation (or is an empty
problem), so no kernel is ever launched; fake device pointers are never
dereferenced.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import weight_quantized_amd as ql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")
LIB = C.CDLL(ql.lib_path)
for name, (res, args) in ql.EXPORTS.items():
    getattr(LIB, name).restype = res
    getattr(LIB, name).argtypes = args

CODES = {}
with open(HEADER) as f:
    for m in re.finditer(r"#define (QL_\w+) \(?(-?\d+)\)?", f.read()):
        CODES[m.group(1)] = int(m.group(2))

FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
MIS = FAKE + 4                 # misaligned
DEF = 0                        # default stream


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ql_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(LIB, n), n
        assert n in ql.EXPORTS, f"binding lacks {n}"


def test_status_strings_and_version():
    for name, code in CODES.items():
        if name.startswith("QL_ERR") or name == "QL_OK":
            assert ql.status_string(code) == name
    assert ql.version() >= 100


def _last():
    return LIB.ql_last_error().decode()


def test_w4a16_gemm_validation():
    g = LIB.ql_w4a16_gemm_path
    E = CODES
    # null weight pointers
    assert g(FAKE, None, FAKE, FAKE, FAKE, 1, 64, 128, 128, None, 0, DEF, 0) == E["QL_ERR_NULL"]
    assert "null" in _last()
    # bad group, k not a multiple of the group, negative sizes
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 16, None, 0, DEF, 0) == E["QL_ERR_GROUP"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 96, 64, None, 0, DEF, 0) == E["QL_ERR_SHAPE"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 64, 128, 128, None, 0, DEF, 0) == E["QL_ERR_SHAPE"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, -64, 128, 128, None, 0, DEF, 0) == E["QL_ERR_SHAPE"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 0, 128, None, 0, DEF, 0) == E["QL_ERR_SHAPE"]
    # misaligned pointers
    assert g(FAKE, MIS, FAKE, FAKE, FAKE, 1, 64, 128, 128, None, 0, DEF, 0) == E["QL_ERR_ALIGN"]
    assert g(MIS, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, None, 0, DEF, 0) == E["QL_ERR_ALIGN"]
    # decode path with m > 64, unknown path
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 64, 128, 128, None, 0, DEF, 1) == E["QL_ERR_UNSUPPORTED"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, None, 0, DEF, 7) == E["QL_ERR_UNSUPPORTED"]
    # split-K shape with missing / short workspace
    need = LIB.ql_w4a16_workspace_bytes(16, 4096, 4096, 128)
    assert need > 0
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 4096, 4096, 128, None, 0, DEF, 0) == E["QL_ERR_WORKSPACE"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 4096, 4096, 128, FAKE, need - 1, DEF, 0) == E["QL_ERR_WORKSPACE"]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 4096, 4096, 128, MIS, need, DEF, 0) == E["QL_ERR_ALIGN"]
    # empty problems succeed without launching; x and y may then be NULL
    assert g(None, FAKE, FAKE, FAKE, None, 0, 64, 128, 128, None, 0, DEF, 0) == E["QL_OK"]
    assert g(None, FAKE, FAKE, FAKE, None, 4, 0, 128, 128, None, 0, DEF, 0) == E["QL_OK"]
    # non-empty with null activations
    assert g(None, FAKE, FAKE, FAKE, FAKE, 1, 64, 128, 128, None, 0, DEF, 2) == E["QL_ERR_NULL"]


def test_workspace_sizes():
    assert LIB.ql_w4a16_workspace_bytes(0, 64, 128, 128) == 0
    assert LIB.ql_w4a16_workspace_bytes(512, 4096, 4096, 64) == 0        # GEMM path needs none
    a = LIB.ql_w4a16_workspace_bytes(1, 4096, 11008, 128)          # few columns: K is split
    b = LIB.ql_w4a16_workspace_bytes(16, 4096, 11008, 128)
    assert 0 < a < b
    assert LIB.ql_w4a16_workspace_bytes(16, 4096, 4096, 128) > 0


def test_workspace_zero_region():
    """The header's zero-region size, the binding's copy of it, and every
    split shape's workspace covering it (two-slice launches keep their
    exchange slots there)."""
    with open(HEADER) as f:
        m = re.search(r"#define QL_W4A16_WS_ZERO_BYTES \((\d+)u \+ \((\d+)u << (\d+)\)\)", f.read())
    assert m, "QL_W4A16_WS_ZERO_BYTES not found"
    zero = int(m.group(1)) + (int(m.group(2)) << int(m.group(3)))
    assert zero == ql.W4A16_WS_ZERO_BYTES
    for shape in [(8, 22016, 4096, 128), (4, 16400, 512, 128), (16, 13824, 5120, 128), (1, 5120, 13824, 128),
                  (1, 4096, 11008, 128), (16, 4096, 11008, 128)]:
        need = LIB.ql_w4a16_workspace_bytes(*shape)
        assert need >= zero, shape


def test_dequant_validation():
    d = LIB.ql_w4a16_dequant
    E = CODES
    assert d(None, FAKE, FAKE, FAKE, None, 64, 128, 128, DEF) == E["QL_ERR_NULL"]
    assert d(FAKE, FAKE, FAKE, None, None, 64, 128, 128, DEF) == E["QL_ERR_NULL"]
    assert d(FAKE, FAKE, FAKE, FAKE, MIS, 64, 128, 128, DEF) == E["QL_ERR_ALIGN"]
    assert d(FAKE, FAKE, FAKE, FAKE, None, 64, 100, 32, DEF) == E["QL_ERR_SHAPE"]
    assert d(FAKE, FAKE, FAKE, FAKE, None, 0, 128, 128, DEF) == E["QL_OK"]


def test_w8a8_validation():
    E = CODES
    q = LIB.ql_w8a8_quant_rmsnorm
    assert q(FAKE, FAKE, 1e-6, FAKE, FAKE, 4, 100, DEF) == E["QL_ERR_SHAPE"]          # k % 8
    assert q(FAKE, FAKE, 1e-6, FAKE, FAKE, 4, 65544, DEF) == E["QL_ERR_UNSUPPORTED"]
    assert q(FAKE, FAKE, float("nan"), FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_VALUE"]
    assert q(FAKE, None, 1e-6, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
    assert q(FAKE, FAKE, 1e-6, MIS, FAKE, 4, 128, DEF) == E["QL_ERR_ALIGN"]
    assert q(None, None, 1e-6, None, None, 0, 128, DEF) == E["QL_OK"]
    gm = LIB.ql_w8a8_gemm
    assert gm(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 100, DEF) == E["QL_ERR_SHAPE"]     # k % 16
    assert gm(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 131088, DEF) == E["QL_ERR_UNSUPPORTED"]
    assert gm(FAKE, None, FAKE, FAKE, FAKE, 4, 64, 128, DEF) == E["QL_ERR_NULL"]
    assert gm(FAKE, FAKE, MIS, FAKE, FAKE, 4, 64, 128, DEF) == E["QL_ERR_ALIGN"]
    assert gm(None, None, None, None, None, 0, 64, 128, DEF) == E["QL_OK"]
    gi = LIB.ql_w8a8_gemm_i32
    assert gi(FAKE, FAKE, None, 4, 64, 128, DEF) == E["QL_ERR_NULL"]
    assert gi(FAKE, FAKE, FAKE, 4, -1, 128, DEF) == E["QL_ERR_SHAPE"]


def test_python_binding_raises():
    with pytest.raises(ql.QLError) as e:
        ql.awq_pack(np.zeros((4, 100), np.float32), 32)
    assert e.value.code == CODES["QL_ERR_SHAPE"]
    with pytest.raises(ql.QLError) as e:
        ql.awq_pack(np.zeros((4, 128), np.float32), 48)
    assert e.value.code == CODES["QL_ERR_GROUP"]


def test_w8a8_fused_validation():
    E = CODES
    a = LIB.ql_w8a8_add_quant_rmsnorm
    assert a(FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE, FAKE, 4, 100, DEF) == E["QL_ERR_SHAPE"]
    assert a(FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE, FAKE, 4, 65544, DEF) == E["QL_ERR_UNSUPPORTED"]
    assert a(FAKE, FAKE, FAKE, float("inf"), FAKE, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_VALUE"]
    assert a(FAKE, None, FAKE, 1e-6, FAKE, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
    assert a(FAKE, FAKE, FAKE, 1e-6, None, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
    assert a(FAKE, FAKE, FAKE, 1e-6, MIS, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_ALIGN"]
    assert a(None, None, None, 1e-6, None, None, None, 0, 128, DEF) == E["QL_OK"]
    p = LIB.ql_w8a8_quant_per_token
    assert p(FAKE, FAKE, FAKE, 4, 100, DEF) == E["QL_ERR_SHAPE"]
    assert p(FAKE, None, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
    assert p(MIS, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_ALIGN"]
    assert p(None, None, None, 0, 128, DEF) == E["QL_OK"]
    g = LIB.ql_w8a8_gemm_ex
    assert g(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 64, 100, DEF) == E["QL_ERR_SHAPE"]
    assert g(FAKE, FAKE, FAKE, FAKE, MIS, None, FAKE, 4, 64, 128, DEF) == E["QL_ERR_ALIGN"]
    assert g(FAKE, FAKE, FAKE, FAKE, None, MIS, FAKE, 4, 64, 128, DEF) == E["QL_ERR_ALIGN"]
    assert g(FAKE, None, FAKE, FAKE, None, None, FAKE, 4, 64, 128, DEF) == E["QL_ERR_NULL"]
    assert g(None, None, None, None, None, None, None, 0, 64, 128, DEF) == E["QL_OK"]


def test_fp8_validation():
    E = CODES
    q = LIB.ql_fp8_quant_rmsnorm
    assert q(FAKE, FAKE, 1e-6, FAKE, FAKE, 4, 100, DEF) == E["QL_ERR_SHAPE"]
    assert q(FAKE, None, 1e-6, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
    assert q(FAKE, FAKE, float("nan"), FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_VALUE"]
    assert q(None, None, 1e-6, None, None, 0, 128, DEF) == E["QL_OK"]
    p = LIB.ql_fp8_quant_per_token
    assert p(FAKE, FAKE, FAKE, 4, 100, DEF) == E["QL_ERR_SHAPE"]
    assert p(MIS, FAKE, FAKE, 4, 128, DEF) == E["QL_ERR_ALIGN"]
    g = LIB.ql_fp8_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 64, 100, DEF) == E["QL_ERR_SHAPE"]       # k % 16
    assert g(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 64, 96, DEF) == E["QL_ERR_UNSUPPORTED"]  # k % 64
    assert g(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, 64, 4096, DEF) == E["QL_ERR_UNSUPPORTED"]  # 4 GiB
    assert g(FAKE, None, FAKE, FAKE, None, None, FAKE, 4, 64, 128, DEF) == E["QL_ERR_NULL"]
    assert g(FAKE, FAKE, FAKE, FAKE, MIS, None, FAKE, 4, 64, 128, DEF) == E["QL_ERR_ALIGN"]
    assert g(None, None, None, None, None, None, None, 0, 64, 128, DEF) == E["QL_OK"]
    w = np.zeros((2, 8), np.float32)
    wq = np.zeros((2, 8), np.uint8)
    ws = np.zeros(2, np.float32)
    w[1, 3] = np.inf
    assert LIB.ql_fp8_quant_weight(w.ctypes.data, 2, 8, wq.ctypes.data, ws.ctypes.data) == E["QL_ERR_VALUE"]


def test_kv_int8_validation():
    E = CODES
    for f in (LIB.ql_kv_quant_int8, LIB.ql_kv_dequant_int8):
        assert f(FAKE, FAKE, FAKE, 4, 48, DEF) == E["QL_ERR_GROUP"]
        assert f(FAKE, FAKE, FAKE, -1, 128, DEF) == E["QL_ERR_SHAPE"]
        assert f(FAKE, None, FAKE, 4, 128, DEF) == E["QL_ERR_NULL"]
        assert f(FAKE, FAKE, MIS, 4, 128, DEF) == E["QL_ERR_ALIGN"]
        assert f(None, None, None, 0, 128, DEF) == E["QL_OK"]


def test_awq_search_validation():
    E = CODES
    f = LIB.ql_awq_search
    t, n, k, g = 4, 64, 256, 64
    need = LIB.ql_awq_search_workspace_bytes(t, n, k, g)
    assert need > 0
    assert LIB.ql_awq_search_workspace_bytes(t, n, 100, g) == 0
    assert LIB.ql_awq_search_workspace_bytes(0, n, k, g) == 0
    assert LIB.ql_awq_search_workspace_bytes(t, n, k, 48) == 0
    err = np.zeros(8)
    best = np.zeros(1, np.int32)
    s = np.zeros(k, np.float32)
    P = (err.ctypes.data, best.ctypes.data, s.ctypes.data, None, None, None)

    def call(x=FAKE, tt=t, w=FAKE, nn=n, kk=k, gg=g, grid=8, ws=FAKE, wsb=need, tail=P):
        return f(x, tt, w, nn, kk, gg, grid, ws, wsb, DEF, *tail)

    assert call(x=None) == E["QL_ERR_NULL"]
    assert call(ws=None) == E["QL_ERR_NULL"]
    assert call(tail=(None,) + P[1:]) == E["QL_ERR_NULL"]
    assert call(gg=48) == E["QL_ERR_GROUP"]
    assert call(kk=100) == E["QL_ERR_SHAPE"]
    assert call(tt=0) == E["QL_ERR_SHAPE"]
    assert call(grid=0) == E["QL_ERR_SHAPE"]
    assert call(grid=1001) == E["QL_ERR_SHAPE"]
    assert call(tt=1 << 20, kk=4096) == E["QL_ERR_UNSUPPORTED"]
    assert call(wsb=need - 1) == E["QL_ERR_WORKSPACE"]
    assert call(ws=MIS) == E["QL_ERR_ALIGN"]


def test_binding_shape_helpers():
    """The binding's operand checks (host logic, no device): packed weights
    must have the layout ql_awq_pack writes for the layer's (n, k, group)."""
    import torch

    n, k, g = 64, 512, 128
    qw = torch.zeros((n, k // 8), dtype=torch.int32)
    sc = torch.zeros((n, k // g), dtype=torch.float16)
    qz = torch.zeros((n, 1), dtype=torch.int32)
    ql._w4_operands(qw, sc, qz, n, k, g)
    for bad in ((qw[:, :-1], sc, qz), (qw, sc[:, :-1], qz), (qw, sc, torch.zeros((n, 2), dtype=torch.int32)),
                (qw[:-1], sc, qz)):
        with pytest.raises(ValueError):
            ql._w4_operands(*bad, n, k, g)
    with pytest.raises(ValueError):
        ql._w4_operands(qw, sc, qz, n, k, 48)
    with pytest.raises(ValueError):
        ql._w4_operands(qw, sc, qz, n, 500, g)
    with pytest.raises(ValueError):
        ql._shape(torch.zeros(3), (4,), "t")


def test_header_is_c99_and_links_from_c(tmp_path):
    """include/qlinear.h is a plain C header: a C99 program (-pedantic,
    warnings as errors) includes it, links against libqlinear and calls the
    entry points that touch no device (version, status strings, workspace
    sizes, argument checks)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r"""
#include <stdio.h>
#include "qlinear.h"
int main(void)
{
    size_t ws = ql_w4a16_workspace_bytes(8, 22016, 4096, 128);
    int rc = ql_w4a16_gemm(0, 0, 0, 0, 0, 1, 64, 128, 128, 0, 0, 0);
    printf("%d|%s|%d|%d\n", ql_version(), ql_status_string(QL_ERR_NULL), (int)(ws >= QL_W4A16_WS_ZERO_BYTES), rc);
    return 0;
}
""")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(ql.lib_path)
    subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lqlinear", "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.strip().split("|")
    assert int(out[0]) == LIB.ql_version()
    assert out[1] == LIB.ql_status_string(CODES["QL_ERR_NULL"]).decode()
    assert out[2] == "1" and int(out[3]) == CODES["QL_ERR_NULL"]
