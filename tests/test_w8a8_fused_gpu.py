"""The steps beside the W8A8 path on the GPU against the oracle: QRMSNorm
with the residual add fused in, per-token int8 quantisation of a plain
activation, and the int8 GEMM epilogue with bias and residual.

Bar: h (fp16 sum), int8 codes and fp32 scales bit-exact; the fp16 GEMM
output bit-exact against the epilogue's fp32 steps applied to the oracle's
exact accumulator, and within 2e-3 of the oracle's fp64 epilogue.
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


def bits(t):
    return t.cpu().numpy().view(np.uint16)


# k reaches one chunk per thread (8, 136), two (4096), eight (16384) and the
# re-reading kernel (16392: 9 chunks per thread, 65536)
@pytest.mark.parametrize("m,k", [(1, 8), (3, 136), (17, 4096), (4, 16384), (5, 16392), (2, 65536)])
def test_add_quant_rmsnorm_bit_exact(ql, m, k):
    x, gamma, _ = workloads.smoothquant_inputs(m=m, k=k, n=1, seed=m + 3 * k)
    rng = np.random.default_rng(m * k)
    r = (rng.standard_normal((m, k)) * 4).astype(np.float16)
    oh, oq, osc = oracle.add_quant_rmsnorm(x, r, gamma, 1e-6)
    h, xq, xs = ql.w8a8_add_quant_rmsnorm(dev(x), dev(r), dev(gamma), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h), oh)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)
    # in place on the residual, then on x
    for which in ("residual", "x"):
        xd, rd = dev(x), dev(r)
        target = rd if which == "residual" else xd
        h2, xq2, xs2 = ql.w8a8_add_quant_rmsnorm(xd, rd, dev(gamma), 1e-6, h_out=target)
        torch.cuda.synchronize()
        assert h2.data_ptr() == target.data_ptr()
        assert np.array_equal(bits(target), oh), which
        assert np.array_equal(xq2.cpu().numpy(), oq), which
        assert np.array_equal(xs2.cpu().numpy().view(np.uint32), osc.view(np.uint32)), which


def test_add_quant_rmsnorm_edge_rows(ql):
    k = 512
    rng = np.random.default_rng(31)
    x = rng.standard_normal((6, k)).astype(np.float16)
    r = rng.standard_normal((6, k)).astype(np.float16)
    r[0] = -x[0]                                          # h = 0: zero token
    x[1] = 0                                              # h = residual
    r[2] = 0                                              # h = x
    x[3] = np.float16(2.0 ** -24)                         # subnormal sums
    r[3] = np.float16(2.0 ** -23)
    r[4, ::2] = np.float16(1e-3) * x[4, ::2]              # addends far below half an ulp
    gamma = rng.uniform(0.5, 1.5, k).astype(np.float16)
    oh, oq, osc = oracle.add_quant_rmsnorm(x, r, gamma, 1e-6)
    h, xq, xs = ql.w8a8_add_quant_rmsnorm(dev(x), dev(r), dev(gamma), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h), oh)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert osc[0] == 0 and not oq[0].any()


@pytest.mark.parametrize("m,k", [(1, 8), (3, 136), (64, 4096), (5, 11008), (2, 65536)])
def test_quant_per_token_bit_exact(ql, m, k):
    rng = np.random.default_rng(7 * m + k)
    x = (rng.standard_normal((m, k)) * rng.uniform(0.01, 100, (m, 1))).astype(np.float16)
    oq, osc = oracle.quant_per_token(x)
    xq, xs = ql.w8a8_quant_per_token(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)


def test_quant_per_token_edge_rows(ql):
    k = 1024
    rng = np.random.default_rng(32)
    x = rng.standard_normal((7, k)).astype(np.float16)
    x[0] = 0                                              # zero token
    x[1] = 0
    x[1, 9] = -3.25                                       # single nonzero
    x[2] = np.float16(65504)                              # largest fp16
    x[3] = np.float16(2.0 ** -24)                         # smallest subnormal
    x[4, ::2] = np.float16(-2.0 ** -24)
    x[5] = np.linspace(-127, 127, k).astype(np.float16)   # quotients near half-integers
    oq, osc = oracle.quant_per_token(x)
    xq, xs = ql.w8a8_quant_per_token(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), oq)


def _epilogue_fp32(acc, xs, ws, bias, res):
    f = (acc.astype(np.float32) * xs[:, None]).astype(np.float32) * ws[None, :]
    if bias is not None:
        f = (f + bias.astype(np.float32)[None, :]).astype(np.float32)
    if res is not None:
        f = (f + res.astype(np.float32)).astype(np.float32)
    return f.astype(np.float16)


# the LDS-staged epilogue of whole tiles (256 x 128, 512 x 256), ragged tiles
# and n % 4 != 0 (element stores), and the register-staged kernel (k % 64)
@pytest.mark.parametrize("m,n,k", [(256, 128, 4096), (512, 256, 512), (300, 260, 1040), (257, 33, 512),
                                   (130, 200, 448)])
def test_gemm_ex_bias_residual(ql, m, n, k):
    rng = np.random.default_rng(11 * m + n + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    bias = (rng.standard_normal(n) * 4).astype(np.float16)
    res = (rng.standard_normal((m, n)) * 4).astype(np.float16)
    acc = oracle.int8_gemm(xq, wq)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    for b, r in ((bias, None), (None, res), (bias, res)):
        y = ql.w8a8_gemm_ex(*d, bias=None if b is None else dev(b), residual=None if r is None else dev(r))
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), _epilogue_fp32(acc, xs, ws, b, r).view(np.uint16))
        ref = oracle.w8a8_forward_ex(xq, xs, wq, ws, bias=b, residual=r)
        err = np.max(np.abs(got.astype(np.float64) - ref)) / np.max(np.abs(ref))
        assert err <= TOL
    # in place: the output is the residual
    rd = dev(res)
    y = ql.w8a8_gemm_ex(*d, bias=dev(bias), residual=rd, out=rd)
    torch.cuda.synchronize()
    assert y.data_ptr() == rd.data_ptr()
    assert np.array_equal(bits(rd), _epilogue_fp32(acc, xs, ws, bias, res).view(np.uint16))


def test_gemm_ex_without_terms_is_gemm(ql):
    rng = np.random.default_rng(33)
    m, n, k = 256, 256, 1024
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    d = [dev(a) for a in (xq, xs, wq, ws)]
    a = ql.w8a8_gemm(*d)
    b = ql.w8a8_gemm_ex(*d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
