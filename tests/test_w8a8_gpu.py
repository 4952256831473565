"""W8A8 (SmoothQuant) HIP path against the oracle (GPU).

Bar: QRMSNorm int8 codes and fp32 scales bit-exact (the mean of squares is
exact on both sides and every other step is one correctly rounded fp32
operation); int32 accumulators bit-exact; fp16 output within 2e-3 of the
oracle's fp64 epilogue relative to max|oracle|.
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


@pytest.mark.parametrize("m,k", [(1, 8), (3, 4096), (17, 1000), (64, 4096), (5, 11008), (2, 65536), (9, 2056),
                                 (4, 4088), (6, 2048)])
def test_quant_rmsnorm_bit_exact(ql, m, k):
    x, gamma, _ = workloads.smoothquant_inputs(m=m, k=k, n=1, seed=m + k)
    xq, xs = ql.w8a8_quant_rmsnorm(dev(x), dev(gamma), 1e-6)
    torch.cuda.synchronize()
    oq, osc = oracle.quant_rmsnorm(x, gamma, 1e-6)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)


def test_quant_rmsnorm_edge_rows(ql):
    k = 512
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, k)).astype(np.float16)
    x[0] = 0                                              # zero token
    x[1] = 0
    x[1, 100] = -2.5                                      # single nonzero
    x[2] = np.float16(65504)                              # largest fp16 everywhere
    x[3] = np.float16(2.0 ** -24)                         # smallest subnormal everywhere
    x[4, ::3] = np.float16(6e-5)                          # subnormal / normal boundary
    x[5] = np.float16(0.5)                                # constant row
    gamma = rng.uniform(0.5, 1.5, k).astype(np.float16)
    gamma[7] = 0
    for eps in (1e-6, 0.0, 1e-2):
        xq, xs = ql.w8a8_quant_rmsnorm(dev(x), dev(gamma), eps)
        torch.cuda.synchronize()
        oq, osc = oracle.quant_rmsnorm(x, gamma, eps)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32)), eps
        assert np.array_equal(xq.cpu().numpy(), oq), eps


# Shapes reach: one k-tile and fewer k-tiles than pipeline stages (64, 192),
# a k-tile count that is not a multiple of the stage count (448 = 7 tiles),
# exactly one full 256x128 tile, ragged m and n, n % 4 != 0 (element stores),
# and k % 64 != 0 (the register-staged kernel: 16, 1040).
@pytest.mark.parametrize("m,n,k", [(1, 64, 16), (5, 64, 128), (130, 200, 4096), (64, 128, 1040), (257, 33, 512),
                                   (256, 128, 64), (300, 260, 192), (64, 128, 448), (512, 256, 640),
                                   (511, 130, 4096)])
def test_gemm_i32_bit_exact_small(ql, m, n, k):
    rng = np.random.default_rng(m + n + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    acc = ql.w8a8_gemm_i32(dev(xq), dev(wq))
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), oracle.int8_gemm(xq, wq))


def test_gemm_i32_saturating_operands(ql):
    k = 4096
    xq = np.full((128, k), 127, np.int8)
    wq = np.full((128, k), 127, np.int8)
    wq[1] = -127
    acc = ql.w8a8_gemm_i32(dev(xq), dev(wq)).cpu().numpy()
    assert (acc[:, 0] == 16129 * k).all() and (acc[:, 1] == -16129 * k).all()


@pytest.mark.parametrize("m,n,k", [(3, 64, 128), (130, 200, 4096), (2048, 512, 4096)])
def test_gemm_fp16_parity_small(ql, m, n, k):
    rng = np.random.default_rng(m * n)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    y = ql.w8a8_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    torch.cuda.synchronize()
    ref = oracle.w8a8_forward(xq, xs, wq, ws)
    assert rel_err(y.cpu().numpy(), ref) <= TOL


def test_config_smoothquant_pipeline(ql):
    """Full W8A8 workload: host smoothing and int8 weights, GPU QRMSNorm and
    int8 GEMM, against the oracle's own pipeline on every output."""
    x, gamma, w = workloads.smoothquant_inputs()
    s, gs, wsm = ql.smooth(x, gamma, w)
    wq, wsc = ql.w8a8_quant_weight(wsm)
    # oracle pipeline, independent of the library's host steps
    os_, ogs, owsm = oracle.smooth(x, gamma, w)
    owq, owsc = oracle.w8_quant_weight(owsm)
    oxq, oxs = oracle.quant_rmsnorm(x, ogs, 1e-6)

    xq, xs = ql.w8a8_quant_rmsnorm(dev(x), dev(gs), 1e-6)
    wq_d, wsc_d = dev(wq), dev(wsc)
    acc = ql.w8a8_gemm_i32(xq, wq_d)
    y = ql.w8a8_gemm(xq, xs, wq_d, wsc_d)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), oxq)
    assert np.array_equal(xs.cpu().numpy(), oxs)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), oracle.int8_gemm(oxq, owq))
    oy = oracle.w8a8_forward(oxq, oxs, owq, owsc)
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, oy) <= TOL


@pytest.mark.parametrize("m,n,k", [(256, 128, 4096), (300, 260, 1040), (2048, 512, 4096)])
def test_gemm_fp16_epilogue_rounding(ql, m, n, k):
    """The fp16 epilogue rounds (float)acc * x_scale to fp32, that times
    w_scale to fp32, then once to fp16 (round to nearest even); checked bit
    for bit from the oracle's exact int32 accumulator."""
    rng = np.random.default_rng(7 * m + n)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    y = ql.w8a8_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    torch.cuda.synchronize()
    acc = oracle.int8_gemm(xq, wq).astype(np.float32)
    want = ((acc * xs[:, None]).astype(np.float32) * ws[None, :]).astype(np.float32).astype(np.float16)
    got = y.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


# Shapes that take the 8-wave 256 x 256 ring with 128-byte k-tiles on 256 CUs:
# whole rounds with whole tiles, ragged m and n inside them, n % 8 != 0 (no
# LDS-staged epilogue) and n % 4 != 0 (element stores), 688 tiles (two full
# rounds and a partial one, ragged last column) and 172 tiles (one partial
# round).  The int32 accumulator and the fp16 epilogue (with bias and
# residual) are checked bit for bit on every output.
@pytest.mark.parametrize("m,n,k", [(2048, 8192, 512), (2000, 8100, 384), (2048, 8098, 256), (4096, 11000, 128),
                                   (1024, 11008, 256)])
def test_gemm_big_tiles(ql, m, n, k):
    rng = np.random.default_rng(m + n + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    bias = (rng.standard_normal(n) * 4).astype(np.float16)
    res = (rng.standard_normal((m, n)) * 4).astype(np.float16)
    rows = np.arange(m)
    acc = ql.w8a8_gemm_i32(dev(xq), dev(wq))
    y = ql.w8a8_gemm_ex(dev(xq), dev(xs), dev(wq), dev(ws), bias=dev(bias), residual=dev(res))
    torch.cuda.synchronize()
    oacc = oracle.int8_gemm(xq, wq, rows=rows)
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), oacc)
    f = (oacc.astype(np.float32) * xs[rows, None]).astype(np.float32) * ws[None, :]
    f = (f + bias.astype(np.float32)[None, :]).astype(np.float32)
    f = (f + res[rows].astype(np.float32)).astype(np.float32)
    assert np.array_equal(y.cpu().numpy()[rows].view(np.uint16), f.astype(np.float16).view(np.uint16))
