"""ql_w4a16_gemm_noalloc through the C ABI (GPU).

The no-allocation variant runs the kernels of ql_w4a16_gemm with the split-K
workspace held by the library, so its output must equal ql_w4a16_gemm's bit
for bit (same kernels, same summation order).  Two calls in a row, the
second on a smaller problem, check that the shared scratch carries nothing
over from one call to the next; the counters it holds must be back at zero
after each call, which the next split-K call depends on.
"""
import ctypes as C

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import weight_quantized_amd as ql
    L = C.CDLL(ql.lib_path)
    for name, (res, args) in ql.EXPORTS.items():
        getattr(L, name).restype = res
        getattr(L, name).argtypes = args
    return L


def _problem(m, n, k, group, seed):
    rng = np.random.default_rng(seed)
    w = workloads.weight(rng, n, k)
    x = workloads.activations(rng, m, k)
    q = oracle.awq_quantize(w, group)
    qw, qz = oracle.awq_pack(q[0], q[1], group)
    sc = q[2].view(np.float16)
    d = [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in (x, qw, sc, qz)]
    return x, (qw, sc, qz), d


def _noalloc(lib, d, m, n, k, group, y):
    stream = torch.cuda.current_stream().cuda_stream
    return lib.ql_w4a16_gemm_noalloc(d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr(),
                                     y.data_ptr(), m, n, k, group, stream)


def _with_workspace(lib, d, m, n, k, group, y):
    need = lib.ql_w4a16_workspace_bytes(m, n, k, group)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.ql_w4a16_gemm(d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr(), y.data_ptr(), m, n,
                           k, group, ws.data_ptr() if need else None, need, stream)
    torch.cuda.synchronize()
    return rc


# pairs of calls, the second smaller: split-K decode (16-row, single-row and
# 32-row kernels, four- and six-wave workgroups, two slices meeting in exchange
# slots), an unsplit launch and the MFMA GEMM (no scratch)
PAIRS = [
    ((16, 4096, 11008, 128), (4, 1100, 4096, 128)),
    ((8, 22016, 4096, 128), (5, 17001, 1024, 64)),
    ((1, 22016, 4096, 128), (1, 4096, 4096, 64)),
    ((32, 4096, 11008, 128), (8, 1000, 2048, 32)),
    ((24, 20000, 2176, 64), (12, 4096, 1024, 128)),
    ((200, 1536, 1024, 64), (40, 256, 512, 128)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm(lib, first, second):
    for i, (m, n, k, group) in enumerate((first, second)):
        x, host, d = _problem(m, n, k, group, seed=m + n + k + i)
        y = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda:0")
        assert _noalloc(lib, d, m, n, k, group, y) == 0, lib.ql_last_error().decode()
        torch.cuda.synchronize()
        ref = torch.empty_like(y)
        assert _with_workspace(lib, d, m, n, k, group, ref) == 0, lib.ql_last_error().decode()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (m, n, k, group)
        rows = np.unique(np.r_[0:8, n - 8:n, np.linspace(0, n - 1, 24).astype(np.int64)])
        want = oracle.w4a16_forward(x, *host, group, rows=rows)
        got = y.cpu().numpy()[:, rows].astype(np.float64)
        assert np.max(np.abs(got - want)) <= TOL * np.max(np.abs(want))


def test_noalloc_repeated_calls_are_identical(lib):
    m, n, k, group = 16, 4096, 11008, 128
    assert lib.ql_w4a16_workspace_bytes(m, n, k, group) > 0      # a split-K launch
    _, _, d = _problem(m, n, k, group, seed=5)
    ys = [torch.empty((m, n), dtype=torch.float16, device="cuda:0") for _ in range(3)]
    for y in ys:
        assert _noalloc(lib, d, m, n, k, group, y) == 0
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])


def test_noalloc_graph_replays_match_eager(lib):
    """The allocation-free entry point captured in a HIP graph (the callers it
    is for): a counter-protocol split launch and a two-slice exchange launch,
    replayed four times with eager work and synchronisation in between; every
    replay equals the eager result bit for bit.  The first call on the device
    (which clears the scratch with a small kernel) runs eagerly, before the
    capture."""
    cases = [(16, 4096, 11008, 128), (8, 17001, 1024, 64)]
    data = []
    for i, (m, n, k, group) in enumerate(cases):
        _, _, d = _problem(m, n, k, group, seed=40 + i)
        y = torch.empty((m, n), dtype=torch.float16, device="cuda:0")
        data.append(((m, n, k, group), d, y))
    eager = []
    for (m, n, k, group), d, y in data:
        assert _noalloc(lib, d, m, n, k, group, y) == 0, lib.ql_last_error().decode()
        torch.cuda.synchronize()
        eager.append(y.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (m, n, k, group), d, y in data:
            assert _noalloc(lib, d, m, n, k, group, y) == 0
    for rep in range(4):
        for _, _, y in data:
            y.fill_(float("nan"))
        (m, n, k, group), d, _ = data[0]
        other = torch.empty((m, n), dtype=torch.float16, device="cuda:0")
        assert _noalloc(lib, d, m, n, k, group, other) == 0        # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, (_, _, y) in zip(eager, data):
            assert torch.equal(e.view(torch.int16), y.view(torch.int16)), rep


def test_noalloc_validation(lib):
    E_NULL, E_GROUP, E_SHAPE = -1, -3, -2
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda:0")
    w = torch.zeros((64, 32), dtype=torch.int32, device="cuda:0")
    s = torch.zeros((64, 2), dtype=torch.float16, device="cuda:0")
    z = torch.zeros((64, 1), dtype=torch.int32, device="cuda:0")
    y = torch.zeros((4, 64), dtype=torch.float16, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    f = lib.ql_w4a16_gemm_noalloc
    assert f(x.data_ptr(), None, s.data_ptr(), z.data_ptr(), y.data_ptr(), 4, 64, 256, 128, stream) == E_NULL
    assert f(x.data_ptr(), w.data_ptr(), s.data_ptr(), z.data_ptr(), y.data_ptr(), 4, 64, 256, 48, stream) == E_GROUP
    assert f(x.data_ptr(), w.data_ptr(), s.data_ptr(), z.data_ptr(), y.data_ptr(), -1, 64, 256, 128, stream) == E_SHAPE
    assert f(None, w.data_ptr(), s.data_ptr(), z.data_ptr(), None, 0, 64, 256, 128, stream) == 0
