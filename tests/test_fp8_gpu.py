"""W8A8 with FP8 E4M3 codes on the GPU against the oracle.

Bar: codes and fp32 scales bit-exact (every step is one correctly rounded
fp32 operation and a cast with ties to even); the fp16 GEMM output within
2e-3 of the oracle's fp64 result relative to max|oracle| (the matrix cores
sum the exact fp8 products in fp32, in their own order).
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


@pytest.mark.parametrize("m,k", [(1, 8), (3, 4096), (17, 1000), (64, 4096), (5, 16392), (2, 65536), (9, 2056),
                                 (4, 4088)])
def test_fp8_quant_rmsnorm_bit_exact(ql, m, k):
    x, gamma, _ = workloads.smoothquant_inputs(m=m, k=k, n=1, seed=m + 5 * k)
    xq, xs = ql.fp8_quant_rmsnorm(dev(x), dev(gamma), 1e-6)
    torch.cuda.synchronize()
    oq, osc = oracle.quant_fp8(x, gamma, 1e-6)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)


def test_fp8_quant_per_token_bit_exact_and_edges(ql):
    k = 1024
    rng = np.random.default_rng(51)
    x = (rng.standard_normal((12, k)) * rng.uniform(0.01, 100, (12, 1))).astype(np.float16)
    x[0] = 0                                              # zero token
    x[1] = 0
    x[1, 9] = -3.25                                       # single nonzero
    x[2] = np.float16(65504)                              # largest fp16
    x[3] = np.float16(2.0 ** -24)                         # smallest subnormal
    x[4] = np.linspace(-448, 448, k).astype(np.float16)  # quotients on the code grid and between
    x[5, ::2] = np.float16(1e-4)                          # codes in the subnormal range
    # scale 3 (max 1344): quotients at the midpoints between e4m3 codes and one
    # fp16 step either side of them, where x * RN(1/3) and the correctly
    # rounded x / 3 can fall on different sides of a rounding boundary
    codes = np.arange(0, 127, dtype=np.uint8)                # every finite positive code
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = np.float16(3.0 * (vals[:-1] + vals[1:]) / 2)
    near = np.concatenate([mids, np.nextafter(mids, np.float16(np.inf)), np.nextafter(mids, np.float16(0))])
    row = np.zeros(k, np.float16)
    row[0] = 1344
    row[1:1 + near.size] = near
    row[1 + near.size:1 + 2 * near.size] = -near
    x[6] = row
    xq, xs = ql.fp8_quant_per_token(dev(x))
    torch.cuda.synchronize()
    oq, osc = oracle.quant_fp8(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


# whole 256 x 128 tiles (LDS-staged epilogue), ragged tiles, n % 4 != 0, a
# shape whose 256 x 256 tiles fill whole rounds of the CUs, and one that runs
# a single partial round of 256 x 256 tiles with ragged m and n
@pytest.mark.parametrize("m,n,k", [(256, 128, 4096), (300, 260, 1024), (257, 33, 512), (64, 128, 448),
                                   (2048, 8192, 512), (1000, 11000, 256)])
def test_fp8_gemm_parity(ql, m, n, k):
    if k % 64:
        k += 64 - k % 64
    rng = np.random.default_rng(m + n + k)
    # codes of realistic size: quantised N(0,1) data, so sums cancel as in a layer
    xq, xs = oracle.quant_fp8(rng.standard_normal((m, k)).astype(np.float16))
    wq, ws = oracle.fp8_quant_weight((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    rows = np.arange(m)
    bias = (rng.standard_normal(n) * 0.5).astype(np.float16)
    res = (rng.standard_normal((m, n)) * 0.5).astype(np.float16)
    ref = oracle.fp8_forward(xq, xs, wq, ws, rows=rows)
    y = ql.fp8_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    y2 = ql.fp8_gemm(dev(xq), dev(xs), dev(wq), dev(ws), bias=dev(bias), residual=dev(res))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got[rows], ref) <= TOL
    ref2 = ref + bias.astype(np.float64)[None, :] + res[rows].astype(np.float64)
    assert rel_err(y2.cpu().numpy()[rows], ref2) <= TOL


def test_fp8_gemm_extreme_codes(ql):
    """All +-448 codes: every product 448^2, the sums exact in fp32 at this k."""
    m, n, k = 64, 128, 256
    xq = np.full((m, k), 0x7E, np.uint8)
    wq = np.full((n, k), 0x7E, np.uint8)
    wq[::2] = 0xFE                                        # -448 on even rows
    xs = np.full(m, 2.0 ** -20, np.float32)
    ws = np.full(n, 2.0 ** -4, np.float32)
    y = ql.fp8_gemm(dev(xq), dev(xs), dev(wq), dev(ws))
    torch.cuda.synchronize()
    want = (448.0 * 448.0 * k * 2.0 ** -24) * np.where(np.arange(n) % 2 == 0, -1.0, 1.0)
    assert np.array_equal(y.cpu().numpy(), np.tile(want, (m, 1)).astype(np.float16))


def test_fp8_smoothquant_layer(ql):
    """The SmoothQuant workload through FP8: smoothing, per-channel FP8
    weights, FP8 QRMSNorm, FP8 GEMM; checked on every output."""
    x, gamma, w = workloads.smoothquant_inputs()
    s, gs, wsm = ql.smooth(x, gamma, w)
    wq, wsc = ql.fp8_quant_weight(wsm)
    xq, xs = ql.fp8_quant_rmsnorm(dev(x), dev(gs), 1e-6)
    y = ql.fp8_gemm(xq, xs, dev(wq), dev(wsc))
    torch.cuda.synchronize()
    oq, osc = oracle.quant_fp8(x, gs, 1e-6)
    assert np.array_equal(xq.cpu().numpy(), oq) and np.array_equal(xs.cpu().numpy(), osc)
    ref = oracle.fp8_forward(oq, osc, wq, wsc)
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= TOL
