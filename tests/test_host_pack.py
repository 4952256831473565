"""Host quantisers of libqlinear against the oracle, bit for bit (CPU only)."""
import numpy as np
import pytest

import oracle
import weight_quantized_amd as ql
import workloads


def _oracle_pack(w, group):
    q, z, s = oracle.awq_quantize(w, group)
    qw, qz = oracle.awq_pack(q, z, group)
    return qw, s, qz


@pytest.mark.parametrize("name,group,rows", [
    ("q_proj", 128, None), ("gate_up", 128, 2048), ("down", 128, 1024),
    ("qkv", 64, 2048), ("13b_up", 32, 1024), ("13b_down", 128, 512), ("13b_down", 32, 512),
])
def test_awq_pack_matches_oracle_on_workloads(name, group, rows):
    w = workloads.config_weight(name)
    if rows is not None:
        w = np.ascontiguousarray(w[:rows])
    qw, sc, qz = ql.awq_pack(w, group)
    oq, os_, oz = _oracle_pack(w, group)
    assert np.array_equal(qw, oq)
    assert np.array_equal(sc.view(np.uint16), os_)
    assert np.array_equal(qz, oz)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_awq_pack_edge_groups(group):
    rng = np.random.default_rng(group + 1)
    k = 8 * group + group   # odd group count: padded zero words
    w = workloads.weight(rng, 40, k, outliers="normal0.3", outlier_frac=0.05)
    w[0] = 0                                  # all-zero rows
    w[1] = np.abs(w[1]) + 1e-3                # strictly positive groups
    w[2] = -np.abs(w[2]) - 1e-3               # strictly negative groups
    w[3, :group] = 7.5e-5                     # tiny range: the 2^-14 scale floor
    w[4] = rng.uniform(-1e4, 1e4, size=k)     # large magnitudes
    w[5, ::2] = 0.5                           # exact ties in w / s
    w[5, 1::2] = -0.25
    qw, sc, qz = ql.awq_pack(w, group)
    oq, os_, oz = _oracle_pack(w, group)
    assert np.array_equal(qw, oq)
    assert np.array_equal(sc.view(np.uint16), os_)
    assert np.array_equal(qz, oz)
    zw = qz.view(np.uint32)
    groups = k // group
    pad = 8 * zw.shape[1] - groups
    assert pad > 0 and ((zw[:, -1] >> (4 * (8 - pad))) == 0).all()


def test_awq_pack_rejects_bad_values_without_writing():
    w = np.ones((4, 128), np.float32)
    w[2, 5] = np.nan
    qw = np.full((4, 16), 7, np.int32)
    sc = np.full((4, 1), 7, np.uint16)
    qz = np.full((4, 1), 7, np.int32)
    import ctypes as C
    lib = C.CDLL(ql.lib_path)
    lib.ql_awq_pack.argtypes = ql.EXPORTS["ql_awq_pack"][1]
    rc = lib.ql_awq_pack(w.ctypes.data, 4, 128, 128, qw.ctypes.data, sc.ctypes.data, qz.ctypes.data)
    assert rc == -7
    assert (qw == 7).all() and (sc == 7).all() and (qz == 7).all()
    with pytest.raises(ql.QLError):
        ql.awq_pack(np.full((2, 128), 3e6, np.float32) * np.float32([[1], [-1]]), 128)


def test_smooth_and_weight_quant_match_oracle():
    x, gamma, w = workloads.smoothquant_inputs(m=512, k=1024, n=768, seed=3)
    gamma[5] = 0
    x[:, 9] = 0
    s, gs, ws = ql.smooth(x, gamma, w)
    os_, ogs, ows = oracle.smooth(x, gamma, w)
    assert np.array_equal(s, os_)
    assert np.array_equal(gs.view(np.uint16), ogs.view(np.uint16))
    assert np.array_equal(ws, ows)
    wq, wsc = ql.w8a8_quant_weight(ws)
    owq, owsc = oracle.w8_quant_weight(ows)
    assert np.array_equal(wq, owq) and np.array_equal(wsc, owsc)


def test_smoothquant_full_workload_matches_oracle():
    x, gamma, w = workloads.smoothquant_inputs()
    s, gs, ws = ql.smooth(x, gamma, w)
    os_, ogs, ows = oracle.smooth(x, gamma, w)
    assert np.array_equal(s, os_) and np.array_equal(gs.view(np.uint16), ogs.view(np.uint16))
    assert np.array_equal(ws, ows)
    wq, wsc = ql.w8a8_quant_weight(ws)
    owq, owsc = oracle.w8_quant_weight(ows)
    assert np.array_equal(wq, owq) and np.array_equal(wsc, owsc)


def test_fp8_weight_quant_matches_oracle():
    """Per-channel FP8 E4M3 weights of the smoothed SmoothQuant workload,
    bit-exact against the oracle, plus rows that reach the subnormal codes,
    a zero row and a single nonzero."""
    x, gamma, w = workloads.smoothquant_inputs(m=64, k=1024, n=96, seed=9)
    _, _, ws = ql.smooth(x, gamma, w)
    ws[0] = 0
    ws[1] = 0
    ws[1, 5] = -7.0
    ws[2] *= np.logspace(-6, 0, ws.shape[1], dtype=np.float32)   # values far below the row maximum
    wq, wsc = ql.fp8_quant_weight(ws)
    oq, osc = oracle.fp8_quant_weight(ws)
    assert np.array_equal(wq, oq) and np.array_equal(wsc.view(np.uint32), osc.view(np.uint32))
    assert not wq[0].any() and wsc[0] == 0 and wq[1, 5] == 0xFE
    assert (wq[2] & 0x78 == 0).any()                           # subnormal codes reached


def test_fp8_weight_quant_full_workload_matches_oracle():
    x, gamma, w = workloads.smoothquant_inputs()
    _, _, ws = ql.smooth(x, gamma, w)
    wq, wsc = ql.fp8_quant_weight(ws)
    oq, osc = oracle.fp8_quant_weight(ws)
    assert np.array_equal(wq, oq) and np.array_equal(wsc.view(np.uint32), osc.view(np.uint32))


def _pack_shapes(count, seed=20261):
    """Seeded (n, k, group) draws: ragged channel counts, odd and even group
    counts (padded zero words or none), k of one group up to a few hundred."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        group = int(rng.choice([32, 64, 128]))
        n = int(rng.integers(1, 300))
        groups = int(rng.integers(1, 40))
        out.append((n, groups * group, group, int(rng.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("n,k,group,seed", _pack_shapes(24))
def test_awq_pack_random_shapes_match_oracle(n, k, group, seed):
    rng = np.random.default_rng(seed)
    w = workloads.weight(rng, n, k, outliers="normal0.3", outlier_frac=0.02)
    qw, sc, qz = ql.awq_pack(w, group)
    oq, os_, oz = _oracle_pack(w, group)
    assert np.array_equal(qw, oq)
    assert np.array_equal(sc.view(np.uint16), os_)
    assert np.array_equal(qz, oz)
