"""Seeded random shapes through every device entry point, against the oracle (GPU).

The other GPU tests pick shapes by hand: the workload configurations, tile
and slice boundaries, ragged edges.  Here the shapes are drawn at random (a
fixed seed, so the set is the same on every run) across the ranges each
kernel choice covers -- 1 to 320 rows for W4A16 (the GEMV, the streamed
decode kernel at 16, 32 and 64 rows, the GEMM), any column count, k any
multiple of the group -- so that a plan or an edge case nobody thought of
still meets the oracle.  Bars as elsewhere: W4A16 and FP8 outputs within
2e-3 of max|oracle| on every output, int8 accumulators and every quantiser's
codes and scales bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def ql():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import weight_quantized_amd
    return weight_quantized_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def rel_err(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / (den if den > 0 else 1.0))


def _w4_shapes(count=80, seed=2024):
    rng = np.random.default_rng(seed)
    buckets = [(1, 3), (4, 16), (17, 32), (33, 64), (65, 320)]
    out = []
    for i in range(count):
        lo, hi = buckets[i % len(buckets)]
        m = int(rng.integers(lo, hi + 1))
        g = int(rng.choice([32, 64, 128]))
        k = g * int(rng.integers(1, 3072 // g + 1))
        n = int(rng.integers(1, 2600))
        out.append((m, n, k, g))
    return out


@pytest.mark.parametrize("m,n,k,g", _w4_shapes())
def test_w4a16_random_shapes(ql, m, n, k, g):
    rng = np.random.default_rng(m * 7919 + n * 31 + k + g)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    qw, sc, qz = ql.awq_pack(w, g)
    d = [dev(a) for a in (qw, sc, qz)]
    # the oracle's unpacking and dequantisation, then the fp64 contraction (numpy's matmul, which the oracle pins
    # hold equal to the oracle's own loop); a few channels through that loop itself
    q, z = oracle.awq_unpack(qw, qz, g)
    _, wd16 = oracle.awq_dequant(q, z, sc, g)
    ref = x.astype(np.float64) @ wd16.astype(np.float64).T
    rows = np.unique(np.linspace(0, n - 1, min(n, 3)).astype(np.int64))
    ref_rows = oracle.w4a16_forward(x, qw, sc, qz, g, rows=rows)
    assert np.allclose(ref[:, rows], ref_rows, rtol=0, atol=1e-9 * max(1.0, float(np.max(np.abs(ref_rows)))))
    paths = [ql.PATH_AUTO] + ([ql.PATH_DECODE, ql.PATH_GEMM] if m <= 64 else [])
    for path in paths:
        y = ql.w4a16_gemm(dev(x), *d, g, path=path).cpu().numpy()
        assert np.isfinite(y).all(), (path,)
        err = rel_err(y, ref)
        assert err <= TOL, (path, err)


def _w8_shapes(count=20, seed=77):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 700)), int(rng.integers(1, 1300)), 16 * int(rng.integers(1, 128)))
            for _ in range(count)]


@pytest.mark.parametrize("m,n,k", _w8_shapes())
def test_w8a8_gemm_random_shapes(ql, m, n, k):
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    acc = ql.w8a8_gemm_i32(dev(xq), dev(wq)).cpu().numpy()
    y = ql.w8a8_gemm(dev(xq), dev(xs), dev(wq), dev(ws)).cpu().numpy()
    oacc = oracle.int8_gemm(xq, wq)
    assert np.array_equal(acc.astype(np.int64), oacc)
    want = ((oacc.astype(np.float32) * xs[:, None]).astype(np.float32) * ws[None, :]).astype(np.float32)
    assert np.array_equal(y.view(np.uint16), want.astype(np.float16).view(np.uint16))


def _tok_shapes(count=10, seed=5):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 40)), 8 * int(rng.integers(1, 3000))) for _ in range(count)]


@pytest.mark.parametrize("m,k", _tok_shapes())
def test_quantisers_random_shapes(ql, m, k):
    x, gamma, _ = workloads.smoothquant_inputs(m=m, k=k, n=1, seed=m + 3 * k)
    xq, xs = ql.w8a8_quant_rmsnorm(dev(x), dev(gamma), 1e-6)
    oq, osc = oracle.quant_rmsnorm(x, gamma, 1e-6)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    fq, fs = ql.fp8_quant_rmsnorm(dev(x), dev(gamma), 1e-6)
    oq8, os8 = oracle.quant_fp8(x, gamma, 1e-6)
    assert np.array_equal(fq.cpu().numpy(), oq8)
    assert np.array_equal(fs.cpu().numpy().view(np.uint32), os8.view(np.uint32))
    tq, ts = ql.w8a8_quant_per_token(dev(x))
    oq1, os1 = oracle.quant_per_token(x)
    assert np.array_equal(tq.cpu().numpy(), oq1)
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), os1.view(np.uint32))


def _f8_shapes(count=8, seed=11):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 600)), int(rng.integers(1, 1200)), 64 * int(rng.integers(1, 40)))
            for _ in range(count)]


@pytest.mark.parametrize("m,n,k", _f8_shapes())
def test_fp8_gemm_random_shapes(ql, m, n, k):
    rng = np.random.default_rng(m + 17 * n + k)
    xq, xs = oracle.quant_fp8(rng.standard_normal((m, k)).astype(np.float16))
    wq, ws = oracle.fp8_quant_weight((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    y = ql.fp8_gemm(dev(xq), dev(xs), dev(wq), dev(ws)).cpu().numpy()
    ref = oracle.fp8_forward(xq, xs, wq, ws)
    assert np.isfinite(y).all()
    assert rel_err(y, ref) <= TOL


def _w4_wide_shapes(count=20, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.integers(1, 65))
        g = int(rng.choice([32, 64, 128]))
        k = g * int(rng.integers(2, 1024 // g + 1))
        n = int(rng.integers(12000, 30000))
        out.append((m, n, k, g))
    return out


# Wide launches (the decode plans' six-wave workgroups, many column blocks,
# split-K at small k) through the ordinary and the allocation-free entry
# points, which must agree bit for bit.
@pytest.mark.parametrize("m,n,k,g", _w4_wide_shapes())
def test_w4a16_wide_random_shapes(ql, m, n, k, g):
    rng = np.random.default_rng(m + 3 * n + k + g)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    qw, sc, qz = ql.awq_pack(w, g)
    d = [dev(a) for a in (qw, sc, qz)]
    q, z = oracle.awq_unpack(qw, qz, g)
    _, wd16 = oracle.awq_dequant(q, z, sc, g)
    ref = x.astype(np.float64) @ wd16.astype(np.float64).T
    xd = dev(x)
    y = ql.w4a16_gemm(xd, *d, g)
    y2 = torch.empty_like(y)
    ql.w4a16_gemm_noalloc(xd, *d, g, out=y2)
    yn = y.cpu().numpy()
    assert np.isfinite(yn).all()
    assert rel_err(yn, ref) <= TOL
    assert torch.equal(y, y2)


def _w4_split_shapes(count=18, seed=4242):
    """Shapes whose decode plans split K in two and meet in exchange slots:
    the streamed kernel at 4-8 rows and 16K-32K channels, plans that would
    split in three or four (4-32 rows, 6K-16K channels, k up to 6144), and
    the GEMV kernel (1-3 rows, 5K-14K channels, k 5K-14K)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        g = int(rng.choice([32, 64, 128]))
        kind = i % 3
        if kind == 0:
            m, n, k = int(rng.integers(4, 9)), int(rng.integers(16400, 32700)), int(rng.integers(512, 4097))
        elif kind == 1:
            m, n, k = int(rng.integers(4, 33)), int(rng.integers(6000, 16000)), int(rng.integers(1024, 6145))
        else:
            m, n, k = int(rng.integers(1, 4)), int(rng.integers(5000, 14000)), int(rng.integers(5120, 14337))
        out.append((m, n, k // g * g, g))
    return out


# Split-in-two launches at larger k than the wide sweep: every call twice on
# one workspace (bit-identical, the exchange slots back at zero), the
# allocation-free entry point bit for bit, and sampled channels (the tail
# included) against the oracle's own loop.
@pytest.mark.parametrize("m,n,k,g", _w4_split_shapes())
def test_w4a16_split_in_two_random_shapes(ql, m, n, k, g):
    rng = np.random.default_rng(m + 5 * n + k + g)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    qw, sc, qz = ql.awq_pack(w, g)
    d = [dev(a) for a in (qw, sc, qz)]
    xd = dev(x)
    ws = torch.zeros(max(ql.w4a16_workspace_bytes(m, n, k, g), 16), dtype=torch.uint8, device="cuda:0")
    y1 = ql.w4a16_gemm(xd, *d, g, workspace=ws).clone()
    y2 = ql.w4a16_gemm(xd, *d, g, workspace=ws)
    y3 = torch.empty_like(y1)
    ql.w4a16_gemm_noalloc(xd, *d, g, out=y3)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()
    yn = y1.cpu().numpy()
    assert np.isfinite(yn).all()
    rows = np.unique(np.concatenate([np.linspace(0, n - 1, 12).astype(np.int64), np.arange(n - 4, n)]))
    ref = oracle.w4a16_forward(x, qw, sc, qz, g, rows=rows)
    assert rel_err(yn[:, rows], ref) <= TOL


@pytest.mark.parametrize("m,k", _tok_shapes(count=8, seed=21))
def test_residual_quantiser_random_shapes(ql, m, k):
    x, gamma, _ = workloads.smoothquant_inputs(m=m, k=k, n=1, seed=2 * m + k)
    rng = np.random.default_rng(m * k)
    r = workloads.activations(rng, m, k)
    h, xq, xs = ql.w8a8_add_quant_rmsnorm(dev(x), dev(r), dev(gamma), 1e-6)
    oh, oq, osc = oracle.add_quant_rmsnorm(x, r, gamma, 1e-6)
    assert np.array_equal(h.cpu().numpy().view(np.uint16), oh)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    fq, fs = ql.fp8_quant_per_token(dev(x))
    oq8, os8 = oracle.quant_fp8(x)
    assert np.array_equal(fq.cpu().numpy(), oq8)
    assert np.array_equal(fs.cpu().numpy().view(np.uint32), os8.view(np.uint32))


@pytest.mark.parametrize("m,n,k", _w8_shapes(count=6, seed=303))
def test_w8a8_epilogue_random_shapes(ql, m, n, k):
    rng = np.random.default_rng(m + n + 5 * k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    bias = (rng.standard_normal(n) * 4).astype(np.float16)
    res = (rng.standard_normal((m, n)) * 4).astype(np.float16)
    y = ql.w8a8_gemm_ex(dev(xq), dev(xs), dev(wq), dev(ws), bias=dev(bias), residual=dev(res)).cpu().numpy()
    oacc = oracle.int8_gemm(xq, wq)
    f = (oacc.astype(np.float32) * xs[:, None]).astype(np.float32) * ws[None, :]
    f = (f + bias.astype(np.float32)[None, :]).astype(np.float32)
    f = (f + res.astype(np.float32)).astype(np.float32)
    assert np.array_equal(y.view(np.uint16), f.astype(np.float16).view(np.uint16))


def _kv_shapes(count=8, seed=8):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        g = int(rng.choice([32, 64, 128]))
        out.append((int(rng.integers(1, 5000)), g))
    return out


@pytest.mark.parametrize("groups,g", _kv_shapes())
def test_kv_int8_random_shapes(ql, groups, g):
    rng = np.random.default_rng(groups * g)
    x = (rng.standard_normal(groups * g) * rng.uniform(0.01, 10.0)).astype(np.float16)
    q, s = ql.kv_quant_int8(dev(x), g)
    oq, osc = oracle.kv_quant_int8(x, g)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    back = ql.kv_dequant_int8(q, s, g).cpu().numpy()
    assert np.array_equal(back.view(np.uint16), oracle.kv_dequant_int8(oq, osc, g))


# Degenerate sizes: one or a few output channels, k of a single group, rows on
# both sides of each kernel boundary (3 | 4, 16 | 17, 32 | 33, 64 | 65).
@pytest.mark.parametrize("n", [1, 2, 17])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("m", [1, 3, 4, 16, 17, 33, 64, 65])
def test_w4a16_tiny_shapes(ql, m, n, g):
    k = g
    rng = np.random.default_rng(m * 100 + n * 10 + g)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    qw, sc, qz = ql.awq_pack(w, g)
    d = [dev(a) for a in (qw, sc, qz)]
    ref = oracle.w4a16_forward(x, qw, sc, qz, g)
    paths = [ql.PATH_AUTO] + ([ql.PATH_DECODE, ql.PATH_GEMM] if m <= 64 else [])
    for path in paths:
        y = ql.w4a16_gemm(dev(x), *d, g, path=path).cpu().numpy()
        assert np.isfinite(y).all(), (path,)
        assert rel_err(y, ref) <= TOL, (path, rel_err(y, ref))
