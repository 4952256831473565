// Host-side quantisers of libqlinear: AWQ-style int4 packing, SmoothQuant
// smoothing and per-channel int8 weights.  These run once per model, offline,
// on the CPU; the per-token work runs in the HIP kernels.
//
// fp16 conversions use the x86 F16C instructions (vcvtps2ph / vcvtph2ps) with
// an explicit rounding mode.  Every fp32 operation is rounded on its own
// (contraction off), so results are reproducible bit for bit.
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "ql_common.hpp"

#pragma clang fp contract(off)

namespace {

inline float half_to_float(uint16_t h) { return _cvtsh_ss(h); }
inline uint16_t float_to_half_rne(float f) { return _cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC); }
inline uint16_t float_to_half_up(float f) { return _cvtss_sh(f, _MM_FROUND_TO_POS_INF | _MM_FROUND_NO_EXC); }

// Run body(lo, hi) over [0, n) split into contiguous ranges on a few threads.
template <class F>
void parallel_rows(int64_t n, F body)
{
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nt = std::max<int64_t>(1, std::min<int64_t>({(int64_t)(hw ? hw : 1), 16, n / 64}));
    if (nt <= 1) {
        body(0, n);
        return;
    }
    std::vector<std::thread> pool;
    int64_t chunk = (n + nt - 1) / nt;
    for (int64_t t = 0; t < nt; ++t) {
        int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
        if (lo < hi)
            pool.emplace_back(body, lo, hi);
    }
    for (auto& th : pool)
        th.join();
}

inline int clamp_code(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace

extern "C" int ql_awq_pack(const float* w, int64_t n, int64_t k, int group, int32_t* qweight,
                           uint16_t* scales, int32_t* qzeros)
{
    ql::clear_error();
    if (!w || !qweight || !scales || !qzeros)
        QL_FAIL(QL_ERR_NULL, "ql_awq_pack: null pointer");
    if (!ql::valid_group(group))
        QL_FAIL(QL_ERR_GROUP, "ql_awq_pack: group %d not in {32, 64, 128}", group);
    if (n < 0 || k <= 0 || k % group)
        QL_FAIL(QL_ERR_SHAPE, "ql_awq_pack: n=%lld k=%lld group=%d", (long long)n, (long long)k, group);

    const int64_t groups = k / group, zwords = (groups + 7) / 8;
    // pass 1: per-group range; reject non-finite input before anything is written
    std::vector<float> gmin((size_t)(n * groups)), gstep((size_t)(n * groups));
    std::atomic<int> bad{0};
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t g = 0; g < groups; ++g) {
                const float* v = w + r * k + g * group;
                float mn = 0.0f, mx = 0.0f;
                for (int i = 0; i < group; ++i) {
                    if (!std::isfinite(v[i]))
                        bad.store(1);
                    mn = std::min(mn, v[i]);
                    mx = std::max(mx, v[i]);
                }
                float step = (mx - mn) / 15.0f;
                if (step < 0x1p-14f)
                    step = 0x1p-14f;            // smallest normal fp16: all-zero groups
                if (step > 65504.0f)
                    bad.store(2);
                gmin[r * groups + g] = mn;
                gstep[r * groups + g] = step;
            }
    });
    if (bad.load() == 1)
        QL_FAIL(QL_ERR_VALUE, "ql_awq_pack: non-finite weight");
    if (bad.load() == 2)
        QL_FAIL(QL_ERR_VALUE, "ql_awq_pack: group range too large for an fp16 scale");

    // pass 2: scale, zero point, codes, packing
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        uint8_t code[128];
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t zi = 0; zi < zwords; ++zi)
                qzeros[r * zwords + zi] = 0;
            for (int64_t g = 0; g < groups; ++g) {
                const float* v = w + r * k + g * group;
                uint16_t sh = float_to_half_up(gstep[r * groups + g]);
                float s = half_to_float(sh);
                int zp = clamp_code((int)std::nearbyint(-gmin[r * groups + g] / s), 0, 15);
                scales[r * groups + g] = sh;
                qzeros[r * zwords + g / 8] |= (int32_t)((uint32_t)zp << (4 * (g % 8)));
                for (int i = 0; i < group; ++i)
                    code[i] = (uint8_t)clamp_code((int)std::nearbyint(v[i] / s) + zp, 0, 15);
                int32_t* out = qweight + r * (k / 8) + g * (group / 8);
                for (int j = 0; j < group / 8; ++j) {
                    uint32_t word = 0;
                    for (int i = 7; i >= 0; --i)
                        word = (word << 4) | code[8 * j + i];
                    out[j] = (int32_t)word;
                }
            }
        }
    });
    return QL_OK;
}

extern "C" int ql_smooth(const uint16_t* x, int64_t rows, const uint16_t* gamma, const float* w,
                         int64_t n, int64_t k, float* s, uint16_t* gamma_smoothed, float* w_smoothed)
{
    ql::clear_error();
    if (!x || !gamma || !w || !s || !gamma_smoothed || !w_smoothed)
        QL_FAIL(QL_ERR_NULL, "ql_smooth: null pointer");
    if (rows < 0 || n < 0 || k <= 0)
        QL_FAIL(QL_ERR_SHAPE, "ql_smooth: rows=%lld n=%lld k=%lld", (long long)rows, (long long)n,
                (long long)k);

    std::vector<float> act(k, 0.0f), wmax(k, 0.0f);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < k; ++j) {
            float v = std::fabs(half_to_float(x[r * k + j]));
            if (!std::isfinite(v))
                QL_FAIL(QL_ERR_VALUE, "ql_smooth: non-finite activation");
            act[j] = std::max(act[j], v);
        }
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            float v = std::fabs(w[r * k + j]);
            if (!std::isfinite(v))
                QL_FAIL(QL_ERR_VALUE, "ql_smooth: non-finite weight");
            wmax[j] = std::max(wmax[j], v);
        }
    for (int64_t j = 0; j < k; ++j) {
        float g = half_to_float(gamma[j]);
        float sj = 1.0f;
        if (act[j] != 0.0f && wmax[j] != 0.0f && g != 0.0f)
            sj = std::sqrt(act[j]) / std::sqrt(wmax[j]);   // alpha = 0.5
        s[j] = sj;
        gamma_smoothed[j] = float_to_half_rne(g / sj);
    }
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t j = 0; j < k; ++j)
                w_smoothed[r * k + j] = w[r * k + j] * s[j];
    });
    return QL_OK;
}

extern "C" int ql_w8a8_quant_weight(const float* w, int64_t n, int64_t k, int8_t* wq, float* w_scale)
{
    ql::clear_error();
    if (!w || !wq || !w_scale)
        QL_FAIL(QL_ERR_NULL, "ql_w8a8_quant_weight: null pointer");
    if (n < 0 || k <= 0)
        QL_FAIL(QL_ERR_SHAPE, "ql_w8a8_quant_weight: n=%lld k=%lld", (long long)n, (long long)k);
    std::vector<float> amax((size_t)n, 0.0f);
    std::atomic<int> bad{0};
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            float a = 0.0f;
            for (int64_t j = 0; j < k; ++j) {
                if (!std::isfinite(w[r * k + j]))
                    bad.store(1);
                a = std::max(a, std::fabs(w[r * k + j]));
            }
            amax[r] = a;
        }
    });
    if (bad.load())
        QL_FAIL(QL_ERR_VALUE, "ql_w8a8_quant_weight: non-finite weight");
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            const float* v = w + r * k;
            float sc = amax[r] / 127.0f;
            w_scale[r] = sc;
            for (int64_t j = 0; j < k; ++j)
                wq[r * k + j] = sc > 0.0f ? (int8_t)clamp_code((int)std::nearbyint(v[j] / sc), -127, 127) : 0;
        }
    });
    return QL_OK;
}

// fp32 -> OCP FP8 E4M3 code, nearest with ties to even (|v| <= 448 here:
// v = w / (max|w| / 448) stays within one fp32 rounding of 448).  Normal
// range: the fp32 pattern rounded to 3 fraction bits by integer addition, the
// exponent rebiased from 127 to 7; below 2^-6, multiples of 2^-9.
static uint8_t e4m3_code(float v)
{
    uint32_t b;
    std::memcpy(&b, &v, sizeof b);
    const uint32_t sgn = (b >> 24) & 0x80u;
    const float a = std::fabs(v);
    uint32_t c;
    if (a >= 448.0f) {
        c = 0x7Eu;
    } else if (a < 0x1p-6f) {
        c = (uint32_t)std::nearbyint(a * 512.0f);
    } else {
        const uint32_t ab = b & 0x7FFFFFFFu;
        const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) & ~0xFFFFFu;
        c = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    }
    return (uint8_t)(sgn | c);
}

extern "C" int ql_fp8_quant_weight(const float* w, int64_t n, int64_t k, uint8_t* wq, float* w_scale)
{
    ql::clear_error();
    if (!w || !wq || !w_scale)
        QL_FAIL(QL_ERR_NULL, "ql_fp8_quant_weight: null pointer");
    if (n < 0 || k <= 0)
        QL_FAIL(QL_ERR_SHAPE, "ql_fp8_quant_weight: n=%lld k=%lld", (long long)n, (long long)k);
    std::vector<float> amax((size_t)n, 0.0f);
    std::atomic<int> bad{0};
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            float a = 0.0f;
            for (int64_t j = 0; j < k; ++j) {
                if (!std::isfinite(w[r * k + j]))
                    bad.store(1);
                a = std::max(a, std::fabs(w[r * k + j]));
            }
            amax[r] = a;
        }
    });
    if (bad.load())
        QL_FAIL(QL_ERR_VALUE, "ql_fp8_quant_weight: non-finite weight");
    parallel_rows(n, [&](int64_t r0, int64_t r1) {
        for (int64_t r = r0; r < r1; ++r) {
            const float* v = w + r * k;
            const float sc = amax[r] / 448.0f;
            w_scale[r] = sc;
            for (int64_t j = 0; j < k; ++j)
                wq[r * k + j] = sc > 0.0f ? e4m3_code(v[j] / sc) : 0;
        }
    });
    return QL_OK;
}
