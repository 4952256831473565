"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these tests compares the oracle with itself.  Each checks a value
printed on the pages (tests/golden/), a closed form, an invariant, a
library routine (NumPy) on the same step, or brute force over exact
rationals on tiny inputs.  CPU only.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            vals[k] = v
    return vals


# --------------------------------------------------------------------------- binary16 codec
def test_f16_decode_exhaustive_vs_numpy():
    h = np.arange(65536, dtype=np.uint16)
    a = oracle.f16_to_f32(h)
    b = h.view(np.float16).astype(np.float32)
    same = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
    assert same.all()


def test_f16_encode_vs_numpy_random_and_midpoints():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # every midpoint between consecutive finite fp16 values, and its float32 neighbours
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)       # exact in float32
    near = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))])
    allx = np.concatenate([x, near, -near, np.float32([65504, 65519.996, 65520, 1e9, 0.0, -0.0])])
    with np.errstate(over="ignore"):
        ref = allx.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16(allx)
    assert np.array_equal(got, ref)


def test_f16_round_up_is_smallest_upper_bound():
    rng = np.random.default_rng(7)
    x = np.exp(rng.uniform(np.log(2.0 ** -14), np.log(60000.0), size=200_000)).astype(np.float32)
    exact = np.arange(0x0400, 0x7BFF, 97, dtype=np.uint16).view(np.float16).astype(np.float32)
    x = np.concatenate([x, exact])
    h = oracle.f32_to_f16_up(x)
    val = h.view(np.float16).astype(np.float32)
    below = (h - 1).astype(np.uint16).view(np.float16).astype(np.float32)
    assert (val >= x).all()
    assert (below < x).all()


# --------------------------------------------------------------------------- P1: worked example
def test_p1_worked_symmetric_example():
    g = _golden("p1_symmetric_example.txt")
    rows, cols = int(g["rows"]), int(g["cols"])
    max_abs = np.float32(float(g["max_abs"]))
    assert rows * cols * 4 == int(g["bytes_fp32"])          # "64 MB" of float32
    rng = np.random.default_rng(0)
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    np.clip(w, -max_abs, max_abs, out=w)
    w[0, 0], w[1, 1] = max_abs, -max_abs                    # max_abs is the page's
    scale, q = oracle.sym_int4(w)
    digits = int(g["scale_printed_digits"])
    assert float(f"{scale:.{digits}g}") == float(g["scale_printed"])
    assert scale == np.float32(max_abs / np.float32(float(g["divisor"])))
    assert q.min() == int(g["q_min"]) and q.max() == int(g["q_max"])
    assert len(np.unique(q)) == int(g["levels"])
    assert q[0, 0] == int(g["q_max"]) and q[1, 1] == int(g["q_min"])
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * float(scale))
    assert err.max() <= float(scale) / 2 * (1 + 2.0 ** -20)


# --------------------------------------------------------------------------- W4A16 quantiser
def _brute_group(wg):
    """Brute force of one group from the definitions (no division formulae):
    smallest fp16 >= max(range/15, 2^-14) by enumeration; the zero point
    minimising |lo - (0 - z) s| over 0..15; per weight the code minimising the
    reconstruction error."""
    lo = min(0.0, float(wg.min()))
    hi = max(0.0, float(wg.max()))
    step = max(np.float32(np.float32(hi - lo) / np.float32(15)), np.float32(2.0 ** -14))
    allh = np.arange(0x0400, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    s = allh[np.searchsorted(allh, step)]
    zs = np.arange(16)
    z = int(zs[np.argmin(np.abs(lo + zs * float(s)))])
    codes = np.arange(16)
    err = np.abs(wg[:, None].astype(np.float64) - (codes[None, :] - z) * float(s))
    return s, z, err.min(axis=1)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantizer_against_brute_force(group):
    rng = np.random.default_rng(group)
    w = workloads.weight(rng, 24, 4 * group, outliers="normal0.3", outlier_frac=0.02)
    w[3, :group] = 0.0                                       # degenerate all-zero group
    w[5, group:2 * group] = np.abs(w[5, group:2 * group])   # one-signed groups
    w[6, :group] = -np.abs(w[6, :group])
    q, z, s = oracle.awq_quantize(w, group)
    sv = s.view(np.float16).astype(np.float32)
    for r in range(w.shape[0]):
        for gi in range(w.shape[1] // group):
            wg = w[r, gi * group:(gi + 1) * group]
            bs, bz, berr = _brute_group(wg)
            assert sv[r, gi] == bs
            assert z[r, gi] == bz
            got = np.abs(wg.astype(np.float64) - (q[r, gi * group:(gi + 1) * group].astype(np.int64) - bz) * float(bs))
            assert (got <= berr + float(bs) * 2.0 ** -20).all()
    assert q[3, :group].max() == 0 and z[3, 0] == 0 and sv[3, 0] == np.float32(2.0 ** -14)


def test_p2_round_trip_bound_on_workloads():
    cases = [("q_proj", 128), ("13b_up", 32)]
    for name, group in cases:
        w = workloads.config_weight(name)
        if name == "13b_up":
            w = w[:2048]
        q, z, s = oracle.awq_quantize(w, group)
        assert q.max() <= 15 and z.max() <= 15
        wd, wd16 = oracle.awq_dequant(q, z, s, group)
        sv = s.view(np.float16).astype(np.float64)
        n, k = w.shape
        err = np.abs(w.astype(np.float64) - wd.astype(np.float64)).reshape(n, k // group, group)
        assert (err <= sv[:, :, None] / 2 * (1 + 2.0 ** -18)).all(), name
        # the fp16 view differs from the exact dequant by at most half an fp16 ulp
        d16 = np.abs(wd16.astype(np.float64) - wd.astype(np.float64))
        ulp = np.spacing(np.abs(wd16)).astype(np.float64)
        assert (d16 <= ulp / 2).all()
        # zero is representable: every all-zero weight reconstructs to exactly 0
        wz = w.copy()
        wz[:, :group] = 0.0
        qz_, zz_, sz_ = oracle.awq_quantize(wz[:4], group)
        wdz, _ = oracle.awq_dequant(qz_, zz_, sz_, group)
        assert (wdz[:, :group] == 0).all()


def test_dequant_matches_float64_definition():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(16, 256), dtype=np.uint8)
    z = rng.integers(0, 16, size=(16, 2), dtype=np.uint8)
    s = (rng.uniform(2.0 ** -14, 0.5, size=(16, 2))).astype(np.float16)
    wd, wd16 = oracle.awq_dequant(q, z, s.view(np.uint16), 128)
    ref = (q.astype(np.float64) - np.repeat(z, 128, axis=1)) * np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.array_equal(wd.astype(np.float64), ref)              # exact in fp32
    assert np.array_equal(wd16, ref.astype(np.float16))             # one RNE rounding


# --------------------------------------------------------------------------- P3: packing
def test_p3_nibble_order_matches_hex_digits():
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2 ** 32, size=(64, 32), dtype=np.uint64).astype(np.uint32)
    zeros = rng.integers(0, 2 ** 32, size=(64, 1), dtype=np.uint64).astype(np.uint32)
    q, z = oracle.awq_unpack(words.view(np.int32), zeros.view(np.int32), 32)
    for r in range(64):
        for j in range(32):
            digits = format(int(words[r, j]), "08x")[::-1]        # least significant digit first
            assert [int(d, 16) for d in digits] == list(q[r, 8 * j:8 * j + 8])
        digits = format(int(zeros[r, 0]), "08x")[::-1]
        assert [int(d, 16) for d in digits] == list(z[r, :8])


def test_p3_pack_unpack_round_trip():
    """pack(unpack(w)) == w.  Every 16-bit pattern appears in both halves of a
    word, each combined with 64 random other halves (8.4M words), so every
    nibble value is seen at every position next to every neighbouring pattern."""
    rng = np.random.default_rng(21)
    half = np.arange(65536, dtype=np.uint32)
    other = rng.integers(0, 65536, size=64, dtype=np.uint32)
    lo_words = (other[:, None] << 16) | half[None, :]
    hi_words = (half[None, :] << 16) | other[:, None]
    words = np.concatenate([lo_words.reshape(-1), hi_words.reshape(-1)]).reshape(-1, 1024)
    zw = words[:, :128].copy()                      # group 8: 1024 zeros per row in 128 words
    q, z = oracle.awq_unpack(words.view(np.int32), zw.view(np.int32), 8)
    assert q.max() <= 15 and z.max() <= 15
    qw, qz = oracle.awq_pack(q, z, 8)
    assert np.array_equal(qw.view(np.uint32), words)
    assert np.array_equal(qz.view(np.uint32), zw)


def test_pack_pads_zero_words():
    # K = 11008, G = 128 -> 86 groups -> 11 words, the last holding 6 zeros and 2 pad nibbles
    rng = np.random.default_rng(2)
    q = rng.integers(0, 16, size=(3, 11008), dtype=np.uint8)
    z = rng.integers(0, 16, size=(3, 86), dtype=np.uint8)
    qw, qz = oracle.awq_pack(q, z, 128)
    assert qz.shape == (3, 11)
    assert ((qz.view(np.uint32)[:, 10] >> 24) == 0).all()
    q2, z2 = oracle.awq_unpack(qw, qz, 128)
    assert np.array_equal(q, q2) and np.array_equal(z, z2)


# --------------------------------------------------------------------------- W4A16 matmul
@pytest.mark.parametrize("m,k,group", [(1, 128, 32), (2, 256, 64), (3, 256, 128)])
def test_p5_w4a16_brute_force_rational(m, k, group):
    rng = np.random.default_rng(m * 1000 + k)
    n = 64
    w = workloads.weight(rng, n, k, outliers="pm0.3", outlier_frac=0.01)
    x = workloads.activations(rng, m, k)
    q, z, s = oracle.awq_quantize(w, group)
    qw, qz = oracle.awq_pack(q, z, group)
    y = oracle.w4a16_forward(x, qw, s.view(np.float16), qz, group)
    _, wd16 = oracle.awq_dequant(q, z, s, group)
    xs = [[Fraction(float(v)) for v in row] for row in x.astype(np.float64)]
    ws = [[Fraction(float(v)) for v in row] for row in wd16.astype(np.float64)]
    for i in range(m):
        for j in range(n):
            exact = sum(a * b for a, b in zip(xs[i], ws[j]))
            bound = k * 2.0 ** -53 * float(sum(abs(a * b) for a, b in zip(xs[i], ws[j]))) * 2
            assert abs(float(exact) - y[i, j]) <= bound + 1e-300


def test_p7_w4a16_matmul_vs_numpy():
    rng = np.random.default_rng(3)
    x = workloads.activations(rng, 5, 1024)
    w = workloads.weight(rng, 96, 1024)
    q, z, s = oracle.awq_quantize(w, 128)
    _, wd16 = oracle.awq_dequant(q, z, s, 128)
    y = oracle.w4a16_matmul(x, wd16)
    ref = x.astype(np.float64) @ wd16.astype(np.float64).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    rows = np.array([95, 0, 17])
    assert np.array_equal(oracle.w4a16_matmul(x, wd16, rows), y[:, rows])


def test_p6_w4a16_closed_forms():
    rng = np.random.default_rng(4)
    k, group, n = 512, 64, 32
    w = workloads.weight(rng, n, k)
    q, z, s = oracle.awq_quantize(w, group)
    qw, qz = oracle.awq_pack(q, z, group)
    _, wd16 = oracle.awq_dequant(q, z, s, group)
    x = np.zeros((k, k), np.float16)
    x[np.arange(k), np.arange(k)] = 1.0                      # one-hot rows
    y = oracle.w4a16_forward(x[:64], qw, s, qz, group)
    assert np.array_equal(y, wd16[:, :64].astype(np.float64).T)
    # every code equal to its zero point -> exactly zero output
    qzq = np.repeat(z, group, axis=1)
    qw2, qz2 = oracle.awq_pack(qzq, z, group)
    x2 = workloads.activations(rng, 3, k)
    assert np.array_equal(oracle.w4a16_forward(x2, qw2, s, qz2, group), np.zeros((3, n)))


# --------------------------------------------------------------------------- W8A8: smoothing
def _sq_constants():
    g = _golden("smoothquant_constants.txt")
    return float(g["alpha"]), int(g["int8_qmax"])


def test_p4_smoothquant_identity_power_of_two_exact():
    alpha, _ = _sq_constants()
    assert alpha == 0.5
    rng = np.random.default_rng(8)
    rows, k, n = 16, 64, 24
    pa = rng.integers(-3, 4, size=k)
    pb = rng.integers(-3, 4, size=k)
    # column maxima a_j = 4^pa, b_j = 4^pb -> s_j = 2^(pa - pb) exactly
    x = (rng.uniform(-1, 1, size=(rows, k)) * 4.0 ** pa).astype(np.float16)
    x[0] = (4.0 ** pa).astype(np.float16)
    w = (rng.uniform(-1, 1, size=(n, k)) * 4.0 ** pb).astype(np.float32)
    w[0] = (4.0 ** pb).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=k).astype(np.float16)
    s, gs, ws = oracle.smooth(x, gamma, w)
    assert np.array_equal(s, (2.0 ** (pa - pb)).astype(np.float32))
    lhs = (x.astype(np.float64) * gs.astype(np.float64)) @ ws.astype(np.float64).T
    rhs = (x.astype(np.float64) * gamma.astype(np.float64)) @ w.astype(np.float64).T
    assert np.array_equal(lhs, rhs)


def test_p4_smoothquant_identity_and_direction_real_scales():
    x, gamma, w = workloads.smoothquant_inputs(m=256, k=512, n=384, seed=1)
    s, gs, ws = oracle.smooth(x, gamma, w)
    a = np.abs(x.astype(np.float64)).max(axis=0)
    b = np.abs(w.astype(np.float64)).max(axis=0)
    # alpha = 0.5 equalises the two column maxima: max|X_j| / s_j == max|W'_j| == sqrt(a_j b_j)
    assert np.allclose(a / s, np.sqrt(a * b), rtol=1e-6)
    assert np.allclose(np.abs(ws.astype(np.float64)).max(axis=0), np.sqrt(a * b), rtol=1e-6)
    # direction: channels with large activations get s > 1 (the norm weight shrinks)
    big = a > 10 * np.median(a)
    assert big.any() and (s[big] > 1).all() and (gs.astype(np.float32)[big] < gamma.astype(np.float32)[big]).all()
    # identity up to the fp16 rounding of gamma' (relative 2^-11 per term) and fp32 of W'
    terms = np.abs(x.astype(np.float64) * gamma.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    lhs = (x.astype(np.float64) * gs.astype(np.float64)) @ ws.astype(np.float64).T
    rhs = (x.astype(np.float64) * gamma.astype(np.float64)) @ w.astype(np.float64).T
    assert (np.abs(lhs - rhs) <= (2.0 ** -11 + 2.0 ** -22) * terms).all()


def test_smoothing_skips_zero_positions():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 32)).astype(np.float16)
    w = rng.standard_normal((16, 32)).astype(np.float32)
    gamma = np.ones(32, np.float16)
    gamma[3] = 0
    x[:, 5] = 0
    w[:, 7] = 0
    s, gs, ws = oracle.smooth(x, gamma, w)
    assert s[3] == 1 and s[5] == 1 and s[7] == 1
    assert np.array_equal(ws[:, 3], w[:, 3]) and gs[3] == 0


# --------------------------------------------------------------------------- W8A8: int8 quantisers
def test_w8_weight_quant_bounds():
    _, qmax = _sq_constants()
    rng = np.random.default_rng(10)
    w = rng.standard_normal((64, 300)).astype(np.float32) * 0.02
    w[7] = 0
    wq, sc = oracle.w8_quant_weight(w)
    assert wq.max() <= qmax and wq.min() >= -qmax
    amax_idx = np.argmax(np.abs(w), axis=1)
    for r in range(64):
        if r == 7:
            assert sc[r] == 0 and not wq[r].any()
            continue
        assert sc[r] == np.float32(np.abs(w[r]).max() / np.float32(qmax))
        assert abs(int(wq[r, amax_idx[r]])) == qmax
        err = np.abs(w[r].astype(np.float64) - wq[r].astype(np.float64) * float(sc[r]))
        assert err.max() <= float(sc[r]) / 2 * (1 + 2.0 ** -20)


def test_sumsq_exact_vs_python_rationals():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 0x7C00, size=(20, 333), dtype=np.uint16)  # finite, positive incl. subnormals
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)
    bits[0, :] = 0x7BFF                                   # all maximal: largest possible squares
    bits[1, :] = 0x0001                                   # all smallest subnormals
    for row in bits:
        exact = sum(Fraction(float(v)) ** 2 for v in row.view(np.float16).astype(np.float64))
        got = oracle.sumsq_exact(row)
        assert Fraction(got, 2 ** 48) == exact


def _nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of a positive rational by bracketing (no division formula)."""
    c = np.float32(float(fr))                              # within one or two ulps
    cands = [c]
    for _ in range(3):
        cands.append(np.nextafter(cands[-1], np.float32(np.inf)))
    d = c
    for _ in range(3):
        d = np.nextafter(d, np.float32(0))
        cands.append(d)
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.float32(v).view(np.uint32)) & 1))
    return np.float32(best)


def test_ratio_to_f32_correct_rounding():
    rng = np.random.default_rng(13)
    for _ in range(3000):
        num = int(rng.integers(1, 2 ** 62)) * int(rng.integers(1, 2 ** 30)) + int(rng.integers(0, 2))
        den = int(rng.integers(1, 1 << 40))
        e2 = int(rng.integers(-60, 0))
        assert oracle.ratio_to_f32(num, den, e2) == _nearest_f32(Fraction(num, den) * Fraction(2) ** e2)
    # exact ties in [2^24, 2^25), where float32 spacing is 2: 2^24 + 1 -> 2^24 (even),
    # 2^24 + 3 -> 2^24 + 4 (even), also reached through a non-trivial denominator
    assert oracle.ratio_to_f32(2 ** 24 + 1, 1, 0) == np.float32(2 ** 24)
    assert oracle.ratio_to_f32(2 ** 24 + 3, 1, 0) == np.float32(2 ** 24 + 4)
    assert oracle.ratio_to_f32(3 * (2 ** 24 + 3), 3, 0) == np.float32(2 ** 24 + 4)
    assert oracle.ratio_to_f32(2 ** 25 + 2, 2, 0) == np.float32(2 ** 24)


def test_quant_rmsnorm_against_float64_rmsnorm():
    _, qmax = _sq_constants()
    x, gamma, _ = workloads.smoothquant_inputs(m=64, k=1024, n=8, seed=2)
    eps = 1e-6
    xq, sc, ms = oracle.quant_rmsnorm(x, gamma, eps, return_ms=True)
    xf = x.astype(np.float64)
    ms64 = (xf ** 2).mean(axis=1)
    assert np.allclose(ms, ms64, rtol=2.0 ** -24)
    y64 = xf / np.sqrt(ms64 + eps)[:, None] * gamma.astype(np.float64)[None, :]
    assert np.allclose(sc, np.abs(y64).max(axis=1) / qmax, rtol=1e-6)
    # dequantised codes sit within half a step (+ fp32 rounding) of the fp64 RMSNorm output
    err = np.abs(xq.astype(np.float64) * sc[:, None].astype(np.float64) - y64)
    assert (err <= sc[:, None] * (0.5 + 1e-4)).all()
    assert (np.abs(xq).max(axis=1) == qmax).all()


def test_quant_rmsnorm_closed_forms():
    k = 256
    x = np.zeros((3, k), np.float16)
    x[0, 17] = 3.0                                       # single nonzero element
    x[2] = np.float16(0.5)
    gamma = np.full(k, 1.25, np.float16)
    xq, sc, ms = oracle.quant_rmsnorm(x, gamma, 1e-6, return_ms=True)
    assert ms[0] == np.float32(9.0 / k)
    assert xq[0, 17] == 127 and np.count_nonzero(xq[0]) == 1
    assert sc[1] == 0 and not xq[1].any()                # all-zero token
    assert (xq[2] == 127).all()                           # constant row -> all at Q_MAX
    # with eps = 0, scaling a token by 2^j leaves codes and scales unchanged
    rng = np.random.default_rng(14)
    xr = rng.standard_normal((4, k)).astype(np.float16)
    a = oracle.quant_rmsnorm(xr, gamma, 0.0)
    b = oracle.quant_rmsnorm((xr.astype(np.float32) * 8).astype(np.float16), gamma, 0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_int8_gemm_vs_python_ints_and_numpy():
    rng = np.random.default_rng(15)
    xq = rng.integers(-127, 128, size=(5, 200), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(7, 200), dtype=np.int8)
    acc = oracle.int8_gemm(xq, wq)
    for i in range(5):
        for j in range(7):
            assert acc[i, j] == sum(int(a) * int(b) for a, b in zip(xq[i], wq[j]))
    assert np.array_equal(acc, xq.astype(np.int64) @ wq.astype(np.int64).T)
    full = np.full((2, 4096), 127, np.int8)
    assert (oracle.int8_gemm(full, full) == 16129 * 4096).all()
    xs = rng.uniform(0.01, 1, 5).astype(np.float32)
    ws = rng.uniform(0.01, 1, 7).astype(np.float32)
    y = oracle.w8a8_forward(xq, xs, wq, ws, rows=np.array([4, 1]), cols=np.array([0, 6]))
    for a, i in enumerate([4, 1]):
        for b, j in enumerate([0, 6]):
            assert y[a, b] == float(acc[i, j]) * float(xs[i]) * float(ws[j])


# --------------------------------------------------------------------------- steps beside the path
def test_add_quant_rmsnorm_sum_is_correctly_rounded():
    """h = fp16(x + residual) equals the exact sum rounded once to binary16,
    by two routes that share nothing with the oracle's codec: NumPy's float16
    addition, and the float64 sum (exact for two binary16 values) converted
    by NumPy."""
    rng = np.random.default_rng(21)
    m, k = 6, 512
    mag = rng.choice(np.array([1e-6, 1e-3, 1.0, 300.0]), (m, k))
    x = (rng.standard_normal((m, k)) * mag).astype(np.float16)
    r = (rng.standard_normal((m, k)) * rng.choice(np.array([1e-6, 1e-3, 1.0, 300.0]), (m, k))).astype(np.float16)
    r[0, :16] = -x[0, :16]                                   # exact cancellation
    r[1, :8] = np.float16(2.0 ** -24)                        # subnormal addend
    gamma = rng.uniform(0.5, 1.5, k).astype(np.float16)
    h, xq, sc = oracle.add_quant_rmsnorm(x, r, gamma)
    assert np.array_equal(h, (x + r).view(np.uint16))
    exact = x.astype(np.float64) + r.astype(np.float64)
    assert np.array_equal(h, exact.astype(np.float16).view(np.uint16))
    assert not h[0, :16].any()


def test_add_quant_rmsnorm_reduces_to_qrmsnorm():
    """A zero residual (either operand zero) reduces step 7 to the pinned
    step 4 on the other operand; h is then that operand bit for bit."""
    x, gamma, _ = workloads.smoothquant_inputs(m=16, k=1024, n=8, seed=3)
    z = np.zeros_like(x)
    for a, b in ((x, z), (z, x)):
        h, xq, sc = oracle.add_quant_rmsnorm(a, b, gamma)
        xq4, sc4 = oracle.quant_rmsnorm(x, gamma)
        assert np.array_equal(h, x.view(np.uint16))
        assert np.array_equal(xq, xq4) and np.array_equal(sc, sc4)


def test_quant_per_token_closed_forms_and_bounds():
    k = 304
    x = np.zeros((4, k), np.float16)
    x[0, 5] = -2.5                                           # single nonzero element
    x[2] = np.float16(0.75)                                  # constant row
    x[3, :] = np.linspace(-4, 4, k).astype(np.float16)
    xq, sc = oracle.quant_per_token(x)
    assert sc[0] == np.float32(2.5) / np.float32(127) and xq[0, 5] == -127 and np.count_nonzero(xq[0]) == 1
    assert sc[1] == 0 and not xq[1].any()                    # all-zero token
    assert (xq[2] == 127).all()
    assert xq[3, 0] == -127 and xq[3, -1] == 127
    # every code reconstructs its input within half a step (plus fp32 rounding of the quotient)
    rng = np.random.default_rng(23)
    xr = (rng.standard_normal((16, k)) * rng.uniform(0.01, 50, (16, 1))).astype(np.float16)
    q, s = oracle.quant_per_token(xr)
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - xr.astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-5)).all()
    assert (np.abs(q).max(axis=1) == 127).all()
    # sign symmetry and power-of-two scaling leave the codes unchanged
    qn, sn = oracle.quant_per_token(-xr)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    q8, s8 = oracle.quant_per_token((xr.astype(np.float32) * 8).astype(np.float16))
    assert np.array_equal(q8, q) and np.array_equal(s8, s * np.float32(8))


def test_w8a8_epilogue_bias_residual_closed_forms():
    rng = np.random.default_rng(24)
    m, n, k = 5, 7, 96
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    xs = rng.uniform(0.01, 1, m).astype(np.float32)
    ws = rng.uniform(0.01, 1, n).astype(np.float32)
    bias = rng.standard_normal(n).astype(np.float16)
    res = rng.standard_normal((m, n)).astype(np.float16)
    # a zero activation leaves exactly the bias, the residual, or their sum
    x0 = np.zeros((m, k), np.int8)
    assert np.array_equal(oracle.w8a8_forward_ex(x0, xs, wq, ws, bias=bias), np.tile(bias.astype(np.float64), (m, 1)))
    assert np.array_equal(oracle.w8a8_forward_ex(x0, xs, wq, ws, residual=res), res.astype(np.float64))
    # no bias and no residual: steps 5-6 as they stand
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    assert np.array_equal(oracle.w8a8_forward_ex(xq, xs, wq, ws), oracle.w8a8_forward(xq, xs, wq, ws))
    # exact rationals with power-of-two scales: every term is exact, so is the float64 sum
    xs2 = np.float32(2.0) ** rng.integers(-8, 0, m).astype(np.float32)
    ws2 = np.float32(2.0) ** rng.integers(-8, 0, n).astype(np.float32)
    y = oracle.w8a8_forward_ex(xq, xs2, wq, ws2, bias=bias, residual=res, rows=np.array([3, 0]),
                               cols=np.array([6, 1, 2]))
    for a, i in enumerate([3, 0]):
        for b, j in enumerate([6, 1, 2]):
            acc = sum(int(p) * int(q) for p, q in zip(xq[i], wq[j]))
            want = (Fraction(acc) * Fraction(float(xs2[i])) * Fraction(float(ws2[j])) + Fraction(float(bias[j]))
                    + Fraction(float(res[i, j])))
            assert Fraction(y[a, b]) == want


# --------------------------------------------------------------------------- FP8 E4M3 (float8_e4m3fn)
def _torch_e4m3(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    import torch
    c = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f32(c)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert got[0x7E] == 448 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_vs_torch_midpoints_and_random():
    vals = oracle.e4m3_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2                        # exact in float32
    pts = np.concatenate([vals, mids, [464.0, 460.0]]).astype(np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    rng = np.random.default_rng(41)
    rnd = (rng.standard_normal(20000) * rng.choice(np.array([1e-3, 0.05, 1.0, 30.0, 150.0]), 20000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 464]
    x = np.concatenate([near, -near, rnd, np.float32([0.0, -0.0])]).astype(np.float32)
    assert np.array_equal(oracle.f32_to_e4m3(x), _torch_e4m3(x))


def test_quant_fp8_closed_forms_and_bound():
    k = 256
    x = np.zeros((4, k), np.float16)
    x[0, 3] = -2.5                                           # single nonzero element
    x[2] = np.float16(0.75)                                  # constant row
    x[3] = np.linspace(-6, 6, k).astype(np.float16)
    q, s = oracle.quant_fp8(x)
    assert s[0] == np.float32(2.5) / np.float32(448) and q[0, 3] == 0xFE and np.count_nonzero(q[0]) == 1
    assert s[1] == 0 and not q[1].any()
    assert (q[2] == 0x7E).all()
    rng = np.random.default_rng(42)
    xr = (rng.standard_normal((16, k)) * rng.uniform(0.01, 50, (16, 1))).astype(np.float16)
    q, s = oracle.quant_fp8(xr)
    dq = oracle.e4m3_to_f32(q).astype(np.float64) * s[:, None].astype(np.float64)
    y = xr.astype(np.float64)
    # half a step of a 3-bit fraction, or half the subnormal step, plus the fp32 quotient's rounding
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert (np.abs(dq - y) <= bound).all()
    assert (np.abs(oracle.e4m3_to_f32(q)).max(axis=1) == 448).all()
    qn, sn = oracle.quant_fp8(-xr)
    assert np.array_equal(qn, np.where(q & 0x7F, q ^ 0x80, q)) and np.array_equal(sn, s)
    q8, s8 = oracle.quant_fp8((xr.astype(np.float32) * 8).astype(np.float16))
    assert np.array_equal(q8, q) and np.array_equal(s8, s * np.float32(8))


def test_quant_fp8_norm_matches_the_pinned_qrmsnorm():
    """With gamma, step 10 normalises exactly as the pinned int8 QRMSNorm: both
    scales come from the same max|y| (one fp32 division by 448, one by 127)."""
    x, gamma, _ = workloads.smoothquant_inputs(m=16, k=1024, n=8, seed=4)
    _, s8 = oracle.quant_fp8(x, gamma)
    _, s1 = oracle.quant_rmsnorm(x, gamma)
    a8 = s8.astype(np.float64) * 448
    a1 = s1.astype(np.float64) * 127
    assert np.allclose(a8, a1, rtol=2.0 ** -22)


def test_fp8_weight_quant_closed_forms():
    w = np.zeros((3, 64), np.float32)
    w[0, 7] = -3.0
    w[2] = np.linspace(-1, 1, 64, dtype=np.float32)
    q, s = oracle.fp8_quant_weight(w)
    assert s[0] == np.float32(3.0) / np.float32(448) and q[0, 7] == 0xFE and np.count_nonzero(q[0]) == 1
    assert s[1] == 0 and not q[1].any()
    assert q[2, 0] == 0xFE and q[2, -1] == 0x7E


def test_fp8_gemm_exact_rationals():
    rng = np.random.default_rng(43)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # no NaN codes
    xq = rng.choice(codes, size=(3, 40))
    wq = rng.choice(codes, size=(5, 40))
    acc = oracle.fp8_forward(xq, None, wq, None)
    xv, wv = oracle.e4m3_to_f32(xq), oracle.e4m3_to_f32(wq)
    for i in range(3):
        for j in range(5):
            want = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[i], wv[j]))
            assert Fraction(acc[i, j]) == want
    xs = rng.uniform(0.01, 1, 3).astype(np.float32)
    ws = rng.uniform(0.01, 1, 5).astype(np.float32)
    y = oracle.fp8_forward(xq, xs, wq, ws, rows=np.array([2]), cols=np.array([4, 0]))
    assert y[0, 0] == acc[2, 4] * float(xs[2]) * float(ws[4]) and y[0, 1] == acc[2, 0] * float(xs[2]) * float(ws[0])


# --------------------------------------------------------------------------- KV cache INT8
def test_kv_quant_closed_forms_and_bound():
    g = 128
    x = np.zeros((4, g), np.float16)
    x[0, 17] = -6.5                                          # single nonzero element
    x[2] = np.float16(0.125)                                 # constant group
    x[3] = np.linspace(-3, 3, g).astype(np.float16)
    q, s = oracle.kv_quant_int8(x, g)
    assert s[0] == np.float32(6.5) / np.float32(127) and q[0, 17] == -127 and np.count_nonzero(q[0]) == 1
    assert s[1] == 0 and not q[1].any()
    assert (q[2] == 127).all() and q[3, 0] == -127 and q[3, -1] == 127
    rng = np.random.default_rng(61)
    xr = (rng.standard_normal((64, g)) * rng.uniform(1e-3, 30, (64, 1))).astype(np.float16)
    for group in (32, 64, 128):
        q, s = oracle.kv_quant_int8(xr, group)
        qs = q.reshape(-1, group).astype(np.float64)
        err = np.abs(qs * s[:, None] - xr.reshape(-1, group).astype(np.float64))
        assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-5)).all()
        assert (np.abs(qs).max(axis=1) == 127).all()
        qn, sn = oracle.kv_quant_int8(-xr, group)
        assert np.array_equal(qn, -q) and np.array_equal(sn, s)
        q8, s8 = oracle.kv_quant_int8((xr.astype(np.float32) * 4).astype(np.float16), group)
        assert np.array_equal(q8, q) and np.array_equal(s8, s * np.float32(4))


def test_kv_dequant_is_the_fp32_product_cast():
    """fp16(fp32(q * scale)) against NumPy's float32 product and float16 cast;
    subnormal and large results included.  Within half an fp16 ulp (plus the
    fp32 rounding) of the exact product."""
    rng = np.random.default_rng(62)
    q = rng.integers(-127, 128, size=(256, 128), dtype=np.int8)
    s = (rng.uniform(0.5, 1.0, 256) * np.float32(2.0) ** rng.integers(-30, 9, 256)).astype(np.float32)
    got = oracle.kv_dequant_int8(q, s, 128)
    want = (q.astype(np.float32) * s[:, None]).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    exact = q.astype(np.float64) * s.astype(np.float64)[:, None]
    val = got.view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(val).astype(np.float16)).astype(np.float64)
    assert (np.abs(val - exact) <= ulp * (0.5 + 2.0 ** -12)).all()


# --------------------------------------------------------------------------- AWQ scale search
def test_f64_to_f16_rounds_once():
    """binary64 -> binary16 against NumPy's direct conversion (which rounds
    the double once), on random magnitudes across the range and on exact
    midpoints between neighbouring binary16 values (ties go to even)."""
    rng = np.random.default_rng(70)
    v = rng.standard_normal(4000) * 2.0 ** rng.integers(-26, 17, 4000)
    h = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    for vals in (v, mids, -mids[::97]):
        got = np.array([oracle.f64_to_f16(a) for a in vals], np.uint16)
        with np.errstate(over="ignore"):          # values past 65520 become inf on both sides
            want = vals.astype(np.float16).view(np.uint16)
        assert np.array_equal(got, want)


def test_awq_scales_closed_forms():
    """act^alpha / w^(1 - alpha) at the ends and the middle of the grid: 1/b,
    sqrt(a/b) and a, within 2 ulp (the fp64 exp/log route rounds once to
    fp32); columns with a zero maximum keep s = 1."""
    rng = np.random.default_rng(71)
    a = (rng.uniform(0.01, 3000.0, 512)).astype(np.float32)
    b = (rng.uniform(1e-4, 0.5, 512)).astype(np.float32)
    a[:3] = [0.0, 5.0, 0.0]
    b[:3] = [0.2, 0.0, 0.0]

    def close(x, y):
        return np.all(np.abs(x.astype(np.float64) - y) <= 2 * np.spacing(np.float32(y)).astype(np.float64))

    with np.errstate(divide="ignore", invalid="ignore"):
        forms = ((0.0, 1.0 / b.astype(np.float64)), (0.5, np.sqrt(a.astype(np.float64) / b)),
                 (1.0, a.astype(np.float64)))
    for alpha, want in forms:
        s = oracle.awq_scales(a, b, alpha)
        assert (s[:3] == 1.0).all()
        assert close(s[3:], want[3:])


def _awq_brute(x, w, group, grid):
    """The search re-derived with NumPy for a tiny case: column maxima,
    x' = fp16(fp32(x) / s), an fp64 matmul rounded once to fp16, squared
    error against the fp64 product of the original operands."""
    xf = x.astype(np.float32)
    a = np.abs(xf).max(axis=0)
    b = np.abs(w).max(axis=0)
    yref = xf.astype(np.float64) @ w.astype(np.float64).T
    errs = []
    for i in range(grid):
        s = oracle.awq_scales(a, b, i / grid)
        q, z, sc = oracle.awq_quantize(w * s[None, :], group)
        _, wd16 = oracle.awq_dequant(q, z, sc, group)
        xs = (xf / s[None, :]).astype(np.float16).astype(np.float64)
        y = (xs @ wd16.astype(np.float64).T).astype(np.float16).astype(np.float64)
        errs.append(float(((y - yref) ** 2).sum()))
    return np.array(errs)


def test_awq_search_brute_force():
    rng = np.random.default_rng(72)
    for t, n, k, group, grid in ((2, 3, 64, 32, 4), (3, 5, 128, 64, 6), (4, 2, 256, 128, 5)):
        x = rng.standard_normal((t, k)).astype(np.float32)
        x[:, rng.choice(k, 2, replace=False)] *= 25
        x = x.astype(np.float16)
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        err, best, s = oracle.awq_search(x, w, group, grid)
        want = _awq_brute(x, w, group, grid)
        assert np.allclose(err, want, rtol=1e-9, atol=0)
        assert best == int(np.argmin(want))
        a = np.abs(x.astype(np.float32)).max(axis=0)
        b = np.abs(w).max(axis=0)
        assert np.array_equal(s, oracle.awq_scales(a, b, best / grid))


def test_awq_search_lossless_round_trip():
    """Without the int4 round trip, (x / s) (W diag(s))^T reproduces x W^T for
    every ratio up to the fp16 roundings of x', W' and y (a scaling applied
    in the wrong direction, or to the wrong axis, fails by orders of
    magnitude); the int4 search's errors are far above that floor and its
    choice is the smallest of them."""
    rng = np.random.default_rng(73)
    t, n, k, group = 16, 64, 256, 64
    x = rng.standard_normal((t, k)).astype(np.float32)
    x[:, rng.choice(k, 3, replace=False)] *= 30
    x = x.astype(np.float16)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    yref = x.astype(np.float64) @ w.astype(np.float64).T
    total = float((yref ** 2).sum())
    err0, _, _ = oracle.awq_search(x, w, group, 10, quant=False)
    assert (err0 / total <= 1e-5).all()
    err, best, _ = oracle.awq_search(x, w, group, 10)
    assert (err / total >= 1e-4).all()
    assert err[best] == err.min() and best == int(np.argmin(err))


def test_awq_search_independent_of_thread_count():
    """The search's error sums do not depend on how many threads run the
    oracle: per-channel partial sums are added in channel order, so runs with
    1 and 3 OpenMP threads give bit-identical errors and the same choice."""
    import json
    import subprocess
    import sys

    code = (
        "import json, numpy as np, oracle\n"
        "rng = np.random.default_rng(74)\n"
        "x = rng.standard_normal((6, 256)).astype(np.float32)\n"
        "x[:, rng.choice(256, 3, replace=False)] *= 30\n"
        "x = x.astype(np.float16)\n"
        "w = (rng.standard_normal((37, 256)) * 0.02).astype(np.float32)\n"
        "err, best, _ = oracle.awq_search(x, w, 64, 8)\n"
        "print(json.dumps({'err': [float(e).hex() for e in err], 'best': best}))\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    runs = []
    for threads in (1, 3):
        env = dict(os.environ, OMP_NUM_THREADS=str(threads), PYTHONPATH=root)
        out = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, check=True, capture_output=True,
                             text=True).stdout
        runs.append(json.loads(out.strip().splitlines()[-1]))
    assert runs[0] == runs[1]
