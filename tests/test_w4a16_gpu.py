"""W4A16 HIP path against the oracle (GPU).

Bar: unpacked codes and fp16 dequantised weights bit-exact; fp16 GEMM output
max|gpu - oracle| / max|oracle| <= 2e-3 (oracle: fp64 accumulation of the
same fp16 dequantised weights).  Every call goes through libqlinear's C ABI.
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


def pack_dev(ql, w, group):
    qw, sc, qz = ql.awq_pack(w, group)
    return (qw, sc, qz), (dev(qw), dev(sc), dev(qz))


def rel_err(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / (den if den > 0 else 1.0))


def oracle_weights64(qw, sc, qz, group):
    """The oracle's dequantised weights fp16((q - z) s), as float64."""
    q, z = oracle.awq_unpack(qw, qz, group)
    _, wd16 = oracle.awq_dequant(q, z, sc, group)
    del q
    return wd16.astype(np.float64)


def oracle_all_channels(x, qw, sc, qz, group, wd64=None):
    """The oracle on every output channel: its unpacking and dequantisation,
    then the fp64 contraction by numpy's matmul, which the oracle pins hold
    equal to the oracle's own fp64 loop to 1e-12 (that loop, an element at a
    time, would take minutes at these sizes).  Tests also check sampled
    channels against the loop itself."""
    if wd64 is None:
        wd64 = oracle_weights64(qw, sc, qz, group)
    return x.astype(np.float64) @ wd64.T


def full_and_sampled(got, x, qw, sc, qz, group, rows, wd64=None):
    """(error over every channel, error over the sampled channels against the
    oracle's own contraction)."""
    ref = oracle_all_channels(x, qw, sc, qz, group, wd64)
    ref_rows = oracle.w4a16_forward(x, qw, sc, qz, group, rows=rows)
    assert np.max(np.abs(ref[:, rows] - ref_rows)) <= 1e-9 * max(np.max(np.abs(ref_rows)), 1e-30)
    return rel_err(got, ref), rel_err(got[:, rows], ref_rows)


def sample_rows(n, seed=0, count=16):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(16, n - 16), size=min(count, max(n - 32, 0)), replace=False) if n > 32 else []
    return np.unique(np.concatenate([np.arange(min(16, n)), np.arange(max(n - 16, 0), n), mid]).astype(np.int64))


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("n,k,group", [(64, 128, 32), (100, 1056, 32), (48, 4096, 128), (64, 4096, 64),
                                       (33, 11008, 128)])
def test_dequant_bit_exact(ql, n, k, group):
    rng = np.random.default_rng(n + k + group)
    w = workloads.weight(rng, n, k, outliers="normal0.3", outlier_frac=0.01)
    w[0, :group] = 0.0
    (qw, sc, qz), d = pack_dev(ql, w, group)
    w16, codes = ql.w4a16_dequant(*d, group, with_codes=True)
    torch.cuda.synchronize()
    oq, oz = oracle.awq_unpack(qw, qz, group)
    _, owd16 = oracle.awq_dequant(oq, oz, sc, group)
    assert np.array_equal(codes.cpu().numpy(), oq)
    assert np.array_equal(w16.cpu().numpy().view(np.uint16), owd16.view(np.uint16))


def test_dequant_bit_exact_q_proj(ql):
    w = workloads.config_weight("q_proj")
    (qw, sc, qz), d = pack_dev(ql, w, 128)
    w16 = ql.w4a16_dequant(*d, 128)
    torch.cuda.synchronize()
    oq, oz = oracle.awq_unpack(qw, qz, 128)
    _, owd16 = oracle.awq_dequant(oq, oz, sc, 128)
    assert np.array_equal(w16.cpu().numpy().view(np.uint16), owd16.view(np.uint16))


# ------------------------------------------------------------------ GEMM, small shapes
SMALL = [
    # m, n, k, group
    (1, 64, 128, 32), (2, 64, 256, 64), (3, 64, 256, 128), (1, 48, 1056, 32), (5, 200, 1024, 64),
    (16, 128, 4096, 128), (17, 64, 512, 32), (31, 96, 2080, 32), (32, 256, 4096, 128),
    (1, 4096, 4096, 128), (8, 1000, 11008, 128),
]


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("m,n,k,group", SMALL)
def test_gemm_small_parity(ql, path, m, n, k, group):
    rng = np.random.default_rng(m * 7 + n * 3 + k + group)
    w = workloads.weight(rng, n, k, outliers="pm0.3")
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y = ql.w4a16_gemm(dev(x), *d, group, path=path)
    torch.cuda.synchronize()
    ref = oracle.w4a16_forward(x, qw, sc, qz, group)
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= TOL


# GEMM path shapes: k % 128 != 0 (1056, 384 with G = 128 and three blocks)
# and an odd number of 128-blocks with G = 128 (1152) take the register-staged
# kernel; the rest the LDS-ring kernel, including an odd block count (1152
# with G = 32, 64), one exactly full 128 x 192 tile, and ragged m and n with
# n % 4 != 0.
@pytest.mark.parametrize("m,n,k,group", [(33, 64, 256, 64), (64, 128, 512, 128), (100, 300, 1056, 32),
                                         (130, 256, 4096, 64), (257, 130, 384, 128), (70, 200, 1152, 32),
                                         (70, 200, 1152, 64), (70, 200, 1152, 128), (128, 192, 512, 64),
                                         (129, 194, 768, 32)])
def test_gemm_path_mid_m(ql, m, n, k, group):
    rng = np.random.default_rng(m + n + k)
    w = workloads.weight(rng, n, k, outliers="normal0.3")
    x = workloads.activations(rng, m, k, outlier_channel_frac=0.01)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y = ql.w4a16_gemm(dev(x), *d, group)
    torch.cuda.synchronize()
    ref = oracle.w4a16_forward(x, qw, sc, qz, group)
    assert rel_err(y.cpu().numpy(), ref) <= TOL


# 128-row launches whose 128 x 192 tiles would leave CUs idle take 128 x 128
# tiles: 200 x 1000 gives 2 x 8 tiles (a ragged last m-tile and n-tile) with K
# split across workgroups; compared on the full output at each group size.
@pytest.mark.parametrize("group", [32, 64, 128])
def test_gemm_128_column_tiles(ql, group):
    m, n, k = 200, 1000, 2048
    rng = np.random.default_rng(m + n + group)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k, outlier_channel_frac=0.01)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y1 = ql.w4a16_gemm(dev(x), *d, group, path=2)
    y2 = ql.w4a16_gemm(dev(x), *d, group, path=2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ref = oracle.w4a16_forward(x, qw, sc, qz, group)
    assert rel_err(y1.cpu().numpy(), ref) <= TOL


# Launches of two or more rounds of 128 x 192 tiles take the 8-wave ring
# kernel: 1000 x 12200 gives 8 x 64 tiles with a ragged last m-tile and
# n-tile; checked on sampled output channels at each group size.
@pytest.mark.parametrize("group", [32, 64, 128])
def test_gemm_eight_wave_ring(ql, group):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    m, n, k = 1000, 12200, 1024
    if -(-m // 128) * -(-n // 192) < 2 * cus:
        pytest.skip("fewer than two rounds of tiles on this device")
    rng = np.random.default_rng(group)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y = ql.w4a16_gemm(dev(x), *d, group, path=2)
    torch.cuda.synchronize()
    rows = sample_rows(n, group)
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    full, sampled = full_and_sampled(got, x, qw, sc, qz, group, rows)
    assert full <= TOL and sampled <= TOL


# GEMM launches whose tiles would leave CUs idle split K into slices whose
# partial tiles the last arrival sums in slice order: 64-row tiles (m <= 64)
# and 128-row tiles, ragged m, n and last slice, every group size; reruns are
# bit-identical and leave the workspace's counters at zero.
@pytest.mark.parametrize("m,n,k,group", [(33, 200, 2048, 128), (64, 1000, 4096, 64), (70, 1000, 4096, 32),
                                         (130, 2000, 3328, 128), (100, 5120, 13824, 32)])
def test_gemm_split_k(ql, m, n, k, group):
    need = ql.w4a16_workspace_bytes(m, n, k, group)
    assert need > 0, "expected a split-K plan"
    rng = np.random.default_rng(m + n + k + group)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k, outlier_channel_frac=0.01)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    y1 = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=2)
    y2 = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()
    got = y1.cpu().numpy()
    assert np.isfinite(got).all()
    full, sampled = full_and_sampled(got, x, qw, sc, qz, group, sample_rows(n, 5))
    assert full <= TOL and sampled <= TOL


# The 32-row decode kernel with 17 to 32 rows (18 column blocks of 64
# channels, the last ragged) and the 64-row kernel with 33 to 64 (eight-wave
# workgroups of 128 channels: 1100 = 8 x 128 + 76), K split into slices,
# 128-channel groups (scale after the MFMA) and 32/64-channel groups (scaled
# fp16 weights); deterministic reruns.
@pytest.mark.parametrize("m,group", [(24, 128), (20, 64), (32, 32), (33, 128), (48, 64), (64, 32), (64, 128)])
def test_decode_17_to_64_rows(ql, m, group):
    n, k = 1100, 11008 if group != 32 else 4096
    rng = np.random.default_rng(m + group)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y1 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    y2 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ref = oracle.w4a16_forward(x, qw, sc, qz, group)
    assert rel_err(y1.cpu().numpy(), ref) <= TOL


# With 128-channel groups the decode kernels multiply the exact integers
# q - z and scale each group's fp32 partial sum; with one nonzero activation
# that partial is exactly q - z and its product with s is exact in fp32, so
# every path must still return the dequantised fp16 weight bit for bit.
@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("path", [1, 2])
def test_gemm_closed_forms(ql, path, group):
    k, n = 1024, 96
    rng = np.random.default_rng(9)
    w = workloads.weight(rng, n, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    w16 = ql.w4a16_dequant(*d, group).cpu().numpy()
    # one-hot rows of x: y[i, :] = w16[:, col_i] exactly
    cols = np.array([0, 1, 7, 8, 31, 32, 127, 128, 500, 1023, 640, 333, 64, 65, 900, 1000])
    x = np.zeros((16, k), np.float16)
    x[np.arange(16), cols] = 1.0
    y = ql.w4a16_gemm(dev(x), *d, group, path=path).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), w16[:, cols].T.copy().view(np.uint16))
    # every code equal to its zero point -> exactly zero
    q, z, s = oracle.awq_quantize(w, group)
    qw2, qz2 = oracle.awq_pack(np.repeat(z, group, axis=1), z, group)
    x2 = workloads.activations(rng, 5, k)
    y2 = ql.w4a16_gemm(dev(x2), dev(qw2), dev(sc), dev(qz2), group, path=path).cpu().numpy()
    assert not y2.any()


# One-hot rows through each decode kernel at 128-channel groups: the GEMV
# kernel (m <= 3), the 16-row kernel, the 32-row kernel (m = 24), six-wave
# workgroups (9-32 rows, N above 64 channels per CU) and the 64-row kernel
# (33-64 rows), with K split into slices where the plan splits it.
@pytest.mark.parametrize("m,n,k", [(1, 1100, 4224), (2, 1100, 4224), (3, 300, 11008), (3, 5120, 13824),
                                   (16, 300, 11008), (24, 1100, 4096), (12, 20000, 512), (32, 20000, 512),
                                   (64, 1100, 4224), (48, 5120, 13824), (40, 20000, 512)])
def test_decode_one_hot_bit_exact_group128(ql, m, n, k):
    group = 128
    rng = np.random.default_rng(m + n + k)
    w = workloads.weight(rng, n, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    w16 = ql.w4a16_dequant(*d, group).cpu().numpy()
    cols = rng.choice(k, size=m, replace=False)
    cols[0] = k - 1
    x = np.zeros((m, k), np.float16)
    x[np.arange(m), cols] = 1.0
    y = ql.w4a16_gemm(dev(x), *d, group, path=1).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), w16[:, cols].T.copy().view(np.uint16))
    # a power-of-two activation scales the exact product by that power (equal
    # values: where the weight is 0 the sum of zero products may be +0 or -0)
    x2 = np.zeros((m, k), np.float16)
    x2[np.arange(m), cols] = -2.0
    y2 = ql.w4a16_gemm(dev(x2), *d, group, path=1).cpu().numpy()
    want = (w16[:, cols].T.astype(np.float32) * np.float32(-2.0)).astype(np.float16)
    assert np.array_equal(y2, want)
    nz = want != 0
    assert np.array_equal(y2[nz].view(np.uint16), want[nz].view(np.uint16))


def test_gemm_empty(ql):
    qw = torch.zeros((64, 16), dtype=torch.int32, device="cuda:0")
    sc = torch.zeros((64, 1), dtype=torch.float16, device="cuda:0")
    qz = torch.zeros((64, 1), dtype=torch.int32, device="cuda:0")
    y = ql.w4a16_gemm(torch.zeros((0, 128), dtype=torch.float16, device="cuda:0"), qw, sc, qz, 128)
    assert y.shape == (0, 64)


# K ending inside a 256-k block, so a slice's last block holds groups past K.
# The scales are read four bytes at a time, so the last channel's last dword
# reaches two bytes past the scale tensor; here those bytes (and the rest of the
# buffer the tensor sits at the front of) hold NaN.  Groups past the slice's
# valid k must never be used: every output stays finite and within the bar.
# (Found by the random shape sweep: M = 16, N = 1471, K = 1504, group 32 put NaN
# in the last column.)
@pytest.mark.parametrize("group,k", [(32, 1504), (64, 1472), (128, 1408)])
@pytest.mark.parametrize("m,path", [(1, 1), (2, 1), (5, 1), (16, 1), (24, 1), (40, 1), (16, 2)])
def test_ragged_k_groups_past_k_unused(ql, m, path, group, k):
    n = 1471
    rng = np.random.default_rng(m + k + group)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), (dq, _, dz) = pack_dev(ql, w, group)
    ng = k // group
    buf = torch.full((n * ng + 64,), float("nan"), dtype=torch.float16, device="cuda:0")
    buf[: n * ng] = dev(sc).reshape(-1)
    ds = buf[: n * ng].view(n, ng)
    y = ql.w4a16_gemm(dev(x), dq, ds, dz, group, path=path).cpu().numpy()
    assert np.isfinite(y).all()
    ref = oracle_all_channels(x, qw, sc, qz, group)
    assert rel_err(y, ref) <= TOL


# Launches of 1-3 rows take the GEMV kernel (one 16-channel tile per
# workgroup, K split among its waves and, where the plan says so, across
# workgroups): a ragged last 256-block (4224 = 16 x 256 + 128; 4160 = 16 x 256
# + 64), a ragged last tile (1100 = 68 x 16 + 12), every group size; K split
# across workgroups because the activation rows exceed their LDS budget
# (3 x 20480 fp16) or because the tiles alone load the CUs unevenly (320 tiles
# for N = 5120).
@pytest.mark.parametrize("m", [1, 2, 3])
@pytest.mark.parametrize("n,k,group", [(1100, 4224, 32), (1100, 4224, 64), (1100, 4224, 128), (1100, 4160, 32),
                                       (1100, 4160, 64), (600, 20480, 128), (5120, 13824, 32)])
def test_decode_gemv(ql, m, n, k, group):
    if k >= 13824:
        assert ql.w4a16_workspace_bytes(m, n, k, group) > 0, "expected K split across workgroups"
    rng = np.random.default_rng(k + group + 7 * m)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y1 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    y2 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ref = oracle.w4a16_forward(x, qw, sc, qz, group)
    assert rel_err(y1.cpu().numpy(), ref) <= TOL


# 9-32 rows on a wide N take six-wave workgroups (96 channels) when that keeps
# every CU at one workgroup: a ragged last workgroup (20000 = 208 x 96 + 32;
# 20001 also ends inside a 16-channel tile) and a ragged K, compared on sampled
# output channels including the tail.  The 16-row ones publish activations
# every second block through a four-slot ring, so block counts that are not a
# multiple of four (1, 5, 7, 9, 13 blocks) run padding blocks.
@pytest.mark.parametrize("m,k,group,n", [(12, 2176, 128, 20000), (24, 2080, 32, 20000), (32, 2176, 64, 20000),
                                         (20, 2176, 128, 20001), (9, 1280, 64, 17000), (16, 3328, 32, 20001),
                                         (13, 256, 128, 16500), (10, 1792, 128, 24577)])
def test_decode_six_wave_workgroups(ql, m, k, group, n):
    rng = np.random.default_rng(m * 3 + k)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    y1 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    y2 = ql.w4a16_gemm(dev(x), *d, group, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    rows = np.unique(np.concatenate([sample_rows(n, 3), np.arange(n - 40, n), np.arange(0, 40)]))
    full, sampled = full_and_sampled(y1.cpu().numpy(), x, qw, sc, qz, group, rows)
    assert full <= TOL and sampled <= TOL


# K split in exactly two slices (2 to 8 rows, 13K-32K channels; two and three
# rows take the streamed kernel instead of the GEMV on such wide layers): the
# slices meet in exchange slots (one atomic swap per pair of output rows)
# instead of arrival counters and partial tiles.  Ragged m (odd rows leave half a pair),
# ragged n (the last 16-channel tile and column block partly outside), ragged
# k (the second slice one block shorter) and every group size; the launch is
# repeated on one workspace (the slots must be back at zero for the second
# call's first arrivals) and all channels are compared with the oracle.
@pytest.mark.parametrize("m,n,k,group", [(4, 16400, 512, 128), (5, 17001, 1024, 64), (7, 20000, 768, 32),
                                         (8, 32700, 1280, 128), (6, 22016, 4096, 128), (8, 22016, 4096, 64),
                                         (2, 17001, 1024, 64), (3, 22016, 4096, 128), (3, 13824, 5120, 32)])
def test_decode_two_slice_exchange(ql, m, n, k, group):
    rng = np.random.default_rng(m * 7 + n + k)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    need = ql.w4a16_workspace_bytes(m, n, k, group)
    assert need >= ql.W4A16_WS_ZERO_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    y1 = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=1).clone()
    y2 = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()
    got = y1.cpu().numpy()
    assert np.isfinite(got).all()
    rows = np.unique(np.concatenate([sample_rows(n, 5), np.arange(n - 20, n)]))
    full, sampled = full_and_sampled(got, x, qw, sc, qz, group, rows)
    assert full <= TOL and sampled <= TOL, (full, sampled)


def test_decode_two_slice_exchange_many_calls(ql):
    """Forty back-to-back calls of each two-slice launch (the streamed kernel
    at gate/up M = 4 and 8, the GEMV kernel at 13B down M = 1) on one
    workspace, without synchronisation between them: arrival orders vary from
    call to call, the outputs must not, and the slots end at zero."""
    group = 128
    for m, n, k in [(4, 22016, 4096), (8, 22016, 4096), (1, 5120, 13824)]:
        rng = np.random.default_rng(m + n)
        w = workloads.weight(rng, n, k)
        _, d = pack_dev(ql, w, group)
        x = dev(workloads.activations(rng, m, k))
        ws = torch.zeros(ql.w4a16_workspace_bytes(m, n, k, group), dtype=torch.uint8, device="cuda:0")
        outs = [ql.w4a16_gemm(x, *d, group, workspace=ws, path=1) for _ in range(40)]
        torch.cuda.synchronize()
        for y in outs[1:]:
            assert torch.equal(y.view(torch.int16), outs[0].view(torch.int16)), (m, n, k)
        assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any(), (m, n, k)


def test_decode_two_slice_exchange_nan_and_zero(ql):
    """Partials that are NaN in one slice only, or zero in both (an all-zero
    activation row): the exchange still tells the first arrival from the
    second, the NaN reaches every output of its row, zero rows give zeros,
    and the slots end at zero."""
    m, n, k, group = 8, 17000, 1024, 128
    rng = np.random.default_rng(77)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    x[2, k - 5] = np.nan          # the second slice's partial of row 2
    x[3, 7] = np.nan              # the first slice's partial of row 3
    x[5] = 0                      # both partials +0
    x[6] = -0.0                   # both partials zero (the products' signs follow the weights)
    (qw, sc, qz), d = pack_dev(ql, w, group)
    ws = torch.zeros(ql.w4a16_workspace_bytes(m, n, k, group), dtype=torch.uint8, device="cuda:0")
    y = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=1)
    y2 = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()
    got = y.cpu().numpy()
    assert np.isnan(got[2]).all() and np.isnan(got[3]).all()
    assert (got[5] == 0).all() and (got[6] == 0).all()
    ok = [0, 1, 4, 7]
    ref = oracle_all_channels(x[ok], qw, sc, qz, group)
    assert rel_err(got[ok], ref) <= TOL


def test_decode_deterministic_and_workspace_left_zero(ql):
    m, n, k, group = 16, 4096, 4096, 128
    rng = np.random.default_rng(4)
    w = workloads.weight(rng, n, k)
    x = dev(workloads.activations(rng, m, k))
    _, d = pack_dev(ql, w, group)
    need = ql.w4a16_workspace_bytes(m, n, k, group)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    y1 = ql.w4a16_gemm(x, *d, group, workspace=ws, path=1).clone()
    y2 = ql.w4a16_gemm(x, *d, group, workspace=ws, path=1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    counters = ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy()
    assert not counters.any()


def test_decode_shared_workspace_across_shapes(ql):
    """One workspace serves calls of different shapes in turn (split-K counters
    and partial sums of one call never alias another call's)."""
    group = 128
    rng = np.random.default_rng(6)
    cases = [(16, 4096, 4096), (1, 22016, 4096), (8, 1000, 11008), (8, 22016, 4096), (16, 22016, 4096),
             (32, 4096, 11008), (5, 17001, 1024)]
    need = max(ql.w4a16_workspace_bytes(m, n, k, group) for m, n, k in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for m, n, k in cases + cases[::-1]:
        w = workloads.weight(rng, n, k)
        x = workloads.activations(rng, m, k)
        (qw, sc, qz), d = pack_dev(ql, w, group)
        y = ql.w4a16_gemm(dev(x), *d, group, workspace=ws, path=1)
        torch.cuda.synchronize()
        rows = sample_rows(n, 1)
        ref = oracle.w4a16_forward(x, qw, sc, qz, group, rows=rows)
        got = y.cpu().numpy()
        assert np.isfinite(got).all()
        assert rel_err(got[:, rows], ref) <= TOL, (m, n, k)
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()


def test_decode_graph_replays_match_eager(ql):
    """Split-K decode launches captured in a HIP graph: every replay, with eager
    work and synchronisation in between, reproduces the eager result exactly
    (the arrival counters reset themselves; no memset nodes are involved)."""
    group = 128
    rng = np.random.default_rng(8)
    cases = [(1, 4096, 4096), (16, 4096, 11008), (6, 17001, 1024)]
    need = max(ql.w4a16_workspace_bytes(m, n, k, group) for m, n, k in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    data = []
    for m, n, k in cases:
        w = workloads.weight(rng, n, k)
        _, d = pack_dev(ql, w, group)
        x = dev(workloads.activations(rng, m, k))
        y = torch.empty((m, n), dtype=torch.float16, device="cuda:0")
        data.append((x, d, y))
    eager = [ql.w4a16_gemm(x, *d, group, workspace=ws, path=1).clone() for x, d, _ in data]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, d, y in data:
            ql.w4a16_gemm(x, *d, group, out=y, workspace=ws, path=1)
    for rep in range(4):
        for _, _, y in data:
            y.fill_(float("nan"))
        ql.w4a16_gemm(data[0][0], *data[0][1], group, workspace=ws, path=1)   # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, (_, _, y) in zip(eager, data):
            assert torch.equal(e, y), rep
    assert not ws[:ql.W4A16_WS_ZERO_BYTES].cpu().numpy().any()


# ------------------------------------------------------------------ full-size configurations
# Every configuration at its full size, compared on every output channel
# (the oracle's dequantised weights and an fp64 contraction) and on sampled
# channels against the oracle's own fp64 loop.
_PACKED = {}


def _packed(ql, name, group, seed=0):
    """Packed weights (host and device) and the oracle's dequantised weights
    of one configuration, kept for the tests that follow with the same one."""
    key = (name, group, seed)
    if key not in _PACKED:
        _PACKED.clear()
        w = workloads.config_weight(name, seed=seed)
        host, d = pack_dev(ql, w, group)
        _PACKED[key] = (host, d, w.shape, oracle_weights64(*host, group))
    return _PACKED[key]


def _config_case(ql, name, m, group, seed=0, rows_seed=0):
    (qw, sc, qz), d, (n, k), wd64 = _packed(ql, name, group, seed)
    x = workloads.config_activations(name, m, k, seed=seed)
    y = ql.w4a16_gemm(dev(x), *d, group)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    return full_and_sampled(got, x, qw, sc, qz, group, sample_rows(n, rows_seed), wd64)


def test_config_q_proj_m1(ql):
    full, sampled = _config_case(ql, "q_proj", 1, 128)
    assert full <= TOL and sampled <= TOL


@pytest.mark.parametrize("m", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_config_llama7b_mlp_decode(ql, name, m):
    full, sampled = _config_case(ql, name, m, 128)
    assert full <= TOL and sampled <= TOL


def test_config_qkv_prefill(ql):
    full, sampled = _config_case(ql, "qkv", 512, 64)
    assert full <= TOL and sampled <= TOL


@pytest.mark.parametrize("m", [1, 8, 64, 256, 1024])
@pytest.mark.parametrize("group", [128, 32])
@pytest.mark.parametrize("name", ["13b_up", "13b_down"])
def test_config_llama13b_sweep(ql, name, m, group):
    full, sampled = _config_case(ql, name, m, group)
    assert full <= TOL and sampled <= TOL
