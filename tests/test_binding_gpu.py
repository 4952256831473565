"""The Python binding's argument checks and its split-K workspace cache (GPU).

Every wrong shape, dtype or device is rejected with ValueError / TypeError
before the C ABI is called, so a mismatched tensor never reaches a kernel.
Decode calls on two streams use separate cached workspaces: their outputs
match the single-stream results and the arrival counters are left at zero.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import weight_quantized_amd
    return weight_quantized_amd


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda:0")


def test_w4a16_rejects_mismatched_operands(ql):
    m, n, k, g = 4, 64, 512, 128
    x = z((m, k), torch.float16)
    qw, sc, qz = z((n, k // 8), torch.int32), z((n, k // g), torch.float16), z((n, 1), torch.int32)
    ql.w4a16_gemm(x, qw, sc, qz, g)          # well-formed: runs
    bad = [
        dict(scales=z((n, k // g + 1), torch.float16)),
        dict(qzeros=z((n, 2), torch.int32)),
        dict(qweight=z((n, k // 8 - 1), torch.int32)),
        dict(out=z((m, n + 1), torch.float16)),
        dict(out=z((m + 1, n), torch.float16)),
        dict(group=64),          # scales then have the wrong width
    ]
    for b in bad:
        args = dict(x=x, qweight=qw, scales=sc, qzeros=qz, group=g)
        args.update(b)
        with pytest.raises(ValueError):
            ql.w4a16_gemm(**args)
    with pytest.raises(TypeError):
        ql.w4a16_gemm(x, qw, sc, qz, g, out=z((m, n), torch.float32))
    with pytest.raises(ValueError):
        ql.w4a16_dequant(qw, z((n, 2 * k // g), torch.float16), qz, g)
    torch.cuda.synchronize()


def test_w8a8_rejects_mismatched_operands(ql):
    m, n, k = 8, 64, 256
    xq, xs = z((m, k), torch.int8), z((m,), torch.float32)
    wq, ws = z((n, k), torch.int8), z((n,), torch.float32)
    ql.w8a8_gemm(xq, xs, wq, ws)
    for args in ((xq, xs, z((n, k + 16), torch.int8), ws), (xq, z((m + 1,), torch.float32), wq, ws),
                 (xq, xs, wq, z((n - 1,), torch.float32))):
        for f in (ql.w8a8_gemm, ql.w8a8_gemm_ex):
            with pytest.raises(ValueError):
                f(*args)
    for f in (ql.w8a8_gemm, ql.w8a8_gemm_ex):
        with pytest.raises(ValueError):
            f(xq, xs, wq, ws, out=z((m, n - 1), torch.float16))
        with pytest.raises(TypeError):
            f(xq, xs, wq, ws, out=z((m, n), torch.float32))
    with pytest.raises(ValueError):
        ql.w8a8_gemm_ex(xq, xs, wq, ws, bias=z((n + 1,), torch.float16))
    with pytest.raises(ValueError):
        ql.w8a8_gemm_i32(xq, wq, out=z((m, n + 1), torch.int32))
    with pytest.raises(ValueError):
        ql.fp8_gemm(z((m, k), torch.uint8), xs, z((n, k), torch.uint8), ws, out=z((m + 1, n), torch.float16))
    x = z((m, k), torch.float16)
    gm = z((k,), torch.float16)
    for f in (ql.w8a8_quant_rmsnorm, ql.fp8_quant_rmsnorm):
        with pytest.raises(ValueError):
            f(x, z((k - 8,), torch.float16))
    with pytest.raises(ValueError):
        ql.w8a8_quant_rmsnorm(x, gm, xq=z((m, k + 8), torch.int8))
    with pytest.raises(ValueError):
        ql.w8a8_quant_rmsnorm(x, gm, x_scale=z((m + 1,), torch.float32))
    with pytest.raises(TypeError):
        ql.fp8_quant_rmsnorm(x, gm, xq=z((m, k), torch.int8))
    with pytest.raises(ValueError):
        ql.w8a8_quant_per_token(x, x_scale=z((m - 1,), torch.float32))
    with pytest.raises(ValueError):
        ql.w8a8_add_quant_rmsnorm(x, z((m, k + 8), torch.float16), gm)
    with pytest.raises(ValueError):
        ql.w8a8_add_quant_rmsnorm(x, x, gm, h_out=z((m, k - 8), torch.float16))
    with pytest.raises(ValueError):
        ql.kv_quant_int8(z((4, 128), torch.float16), 128, scale=z((5,), torch.float32))
    with pytest.raises(ValueError):
        ql.kv_dequant_int8(z((4, 128), torch.int8), z((3,), torch.float32), 128)
    torch.cuda.synchronize()


def test_decode_on_two_streams(ql):
    """Split-K decode launches on two streams without explicit workspaces:
    each stream gets its own cached workspace, so concurrent launches do not
    share arrival counters, partial sums or exchange slots (one launch split
    eight ways through counters, one split in two that exchanges)."""
    group = 128
    rng = np.random.default_rng(11)
    cases = [(8, 4096, 11008), (5, 17001, 1024)]
    data = []
    for m, n, k in cases:
        w = workloads.weight(rng, n, k)
        qw, sc, qz = ql.awq_pack(w, group)
        d = [torch.from_numpy(a).to("cuda:0") for a in (qw, sc, qz)]
        x = torch.from_numpy(workloads.activations(rng, m, k)).to("cuda:0")
        data.append((x, d))
    ref = [ql.w4a16_gemm(x, *d, group, path=1).clone() for x, d in data]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for rep in range(6):
        for i, (s, (x, d)) in enumerate(zip(streams, data)):
            with torch.cuda.stream(s):
                outs[i].append(ql.w4a16_gemm(x, *d, group, path=1))
    torch.cuda.synchronize()
    for i in range(2):
        for y in outs[i]:
            assert torch.equal(y, ref[i])
    keys = [k for k in ql._workspaces if k[2] in (streams[0].cuda_stream, streams[1].cuda_stream)]
    assert len(keys) == 2
    for key in keys:
        assert not ql._workspaces[key][:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()
