"""KV-cache INT8 group quantisation on the GPU against the oracle.

Bar: codes, scales and dequantised fp16 bit-exact (each step is one
correctly rounded fp32 operation, an integer rounding or a cast).
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import weight_quantized_amd
    return weight_quantized_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


# a LLaMA-7B layer's K cache slice [tokens, heads, head_dim], odd group counts
@pytest.mark.parametrize("shape,group", [((1, 32, 128), 128), ((37, 32, 128), 128), ((5, 8, 128), 64),
                                         ((3, 1, 96), 32), ((1024, 32, 128), 128)])
def test_kv_quant_dequant_bit_exact(ql, shape, group):
    rng = np.random.default_rng(sum(shape) + group)
    x = (rng.standard_normal(shape) * rng.uniform(0.01, 20, shape[:-1] + (1,))).astype(np.float16)
    x.reshape(-1)[:group] = 0                              # a zero group
    x.reshape(-1)[group + 3] = np.float16(-65504)          # a group with the largest fp16
    q, s = ql.kv_quant_int8(dev(x), group)
    out = ql.kv_dequant_int8(q, s, group)
    torch.cuda.synchronize()
    oq, osc = oracle.kv_quant_int8(x, group)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.kv_dequant_int8(oq, osc, group))


def test_kv_quant_ties_and_subnormals(ql):
    """Values whose quotients fall on and next to half-integers, and groups of
    fp16 subnormals."""
    g = 128
    base = (np.arange(-63, 65, dtype=np.float64) + 0.5)    # k + 1/2 steps of the scale
    x = np.stack([base * 2.0 ** -3, base * 2.0 ** -20, np.full(g, 2.0 ** -24)]).astype(np.float16)
    x[0, -1] = np.float16(127 * 2.0 ** -3)                 # absmax so scale = 2^-3 exactly
    q, s = ql.kv_quant_int8(dev(x), g)
    torch.cuda.synchronize()
    oq, osc = oracle.kv_quant_int8(x, g)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), osc)
