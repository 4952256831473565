// Host-side quantisers of libqlinear: AWQ-style int4 packing, the AWQ scale
// search, SmoothQuant smoothing and per-channel int8 weights.  These run once
// per model, offline, on the CPU (the scale search scores each candidate with
// the device GEMM); the per-token work runs in the HIP kernels.
//
// fp16 conversions use the x86 F16C instructions (vcvtps2ph / vcvtph2ps) with
// an explicit rounding mode.  Every fp32 operation is rounded on its own
// (contraction off), so results are reproducible bit for bit.
#include <hip/hip_runtime_api.h>
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

// ---------------------------------------------------------------------------
// AWQ scale search (LMDeploy walkthrough, section 2: scales chosen from sampled
// activations to minimise the error of the product; LMDeploy W8A8 guide,
// source analysis of the smoothing: coefficient act^alpha / w^(1 - alpha),
// with per-layer ratios searched in calibration when the scale search is on).
// The grid runs on the host, each candidate's quantised product on the
// device through ql_w4a16_gemm; the unquantised reference is an fp64 host
// product computed once.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kAwqAlign = 256;
inline size_t awq_align(size_t v) { return (v + kAwqAlign - 1) & ~(kAwqAlign - 1); }

struct AwqLayout {
    size_t x, qw, sc, qz, y, ws, ws_bytes, total;
};

AwqLayout awq_layout(int64_t t, int64_t n, int64_t k, int group)
{
    AwqLayout L{};
    size_t off = 0;
    L.x = off;
    off = awq_align(off + (size_t)(t * k) * 2);
    L.qw = off;
    off = awq_align(off + (size_t)(n * (k / 8)) * 4);
    L.sc = off;
    off = awq_align(off + (size_t)(n * (k / group)) * 2);
    L.qz = off;
    off = awq_align(off + (size_t)(n * ((k / group + 7) / 8)) * 4);
    L.y = off;
    off = awq_align(off + (size_t)(t * n) * 2);
    L.ws = off;
    L.ws_bytes = ql_w4a16_workspace_bytes(t, n, k, group);
    off = awq_align(off + L.ws_bytes);
    L.total = off;
    return L;
}

// s_j = act_j^alpha / w_j^(1 - alpha), evaluated as exp(alpha ln a - (1 - alpha) ln b)
// in fp64 and rounded once to fp32; 1 where either maximum is zero.
void awq_ratio_scales(const std::vector<float>& a, const std::vector<float>& b, double alpha, float* s)
{
    for (size_t j = 0; j < a.size(); ++j)
        s[j] = (a[j] == 0.0f || b[j] == 0.0f)
                   ? 1.0f
                   : (float)std::exp(alpha * std::log((double)a[j]) - (1.0 - alpha) * std::log((double)b[j]));
}

int awq_hip(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        QL_FAIL(QL_ERR_HIP, "ql_awq_search: %s: %s", what, hipGetErrorString(e));
    return QL_OK;
}

}  // namespace

extern "C" size_t ql_awq_search_workspace_bytes(int64_t t, int64_t n, int64_t k, int group)
{
    if (t <= 0 || n <= 0 || k <= 0 || !ql::valid_group(group) || k % group)
        return 0;
    return awq_layout(t, n, k, group).total;
}

extern "C" int ql_awq_search(const uint16_t* x, int64_t t, const float* w, int64_t n, int64_t k, int group, int grid,
                             void* workspace, size_t workspace_bytes, void* stream, double* err, int* best,
                             float* s_best, int32_t* qweight, uint16_t* scales, int32_t* qzeros)
{
    ql::clear_error();
    const char* who = "ql_awq_search";
    if (!x || !w || !err || !best || !s_best || !workspace)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::valid_group(group))
        QL_FAIL(QL_ERR_GROUP, "%s: group %d not in {32, 64, 128}", who, group);
    if (t <= 0 || n <= 0 || k <= 0 || k % group || grid < 1 || grid > 1000)
        QL_FAIL(QL_ERR_SHAPE, "%s: t=%lld n=%lld k=%lld group=%d grid=%d", who, (long long)t, (long long)n,
                (long long)k, group, grid);
    if (t * k >= (1LL << 30) || n * k >= (1LL << 32) || t * n >= (1LL << 30))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: t=%lld n=%lld k=%lld too large", who, (long long)t, (long long)n,
                (long long)k);
    const AwqLayout L = awq_layout(t, n, k, group);
    if (workspace_bytes < L.total)
        QL_FAIL(QL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, L.total, workspace_bytes);
    if (!ql::aligned16(workspace))
        QL_FAIL(QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
    char* dws = static_cast<char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ng = k / group, zw = (ng + 7) / 8;

    // 1. column maxima and the fp64 reference product x w^T
    std::vector<float> xf((size_t)(t * k)), a((size_t)k, 0.0f), b((size_t)k, 0.0f);
    for (int64_t i = 0; i < t * k; ++i)
        xf[(size_t)i] = half_to_float(x[i]);
    for (int64_t i = 0; i < t; ++i)
        for (int64_t j = 0; j < k; ++j)
            a[(size_t)j] = std::max(a[(size_t)j], std::fabs(xf[(size_t)(i * k + j)]));
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j) {
            const float v = w[r * k + j];
            if (!std::isfinite(v))
                QL_FAIL(QL_ERR_VALUE, "%s: non-finite weight at (%lld, %lld)", who, (long long)r, (long long)j);
            b[(size_t)j] = std::max(b[(size_t)j], std::fabs(v));
        }
    std::vector<double> yref((size_t)(t * n));
    parallel_rows(n, [&](int64_t lo, int64_t hi) {
        for (int64_t r = lo; r < hi; ++r)
            for (int64_t i = 0; i < t; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j)
                    acc += (double)xf[(size_t)(i * k + j)] * (double)w[r * k + j];
                yref[(size_t)(i * n + r)] = acc;
            }
    });

    // 2. the grid: smooth, quantise, run the int4 product on the device, score
    std::vector<float> s((size_t)k), ws((size_t)(n * k));
    std::vector<int32_t> qw((size_t)(n * (k / 8))), qz((size_t)(n * zw));
    std::vector<uint16_t> sc((size_t)(n * ng)), xs((size_t)(t * k)), y((size_t)(t * n));
    int bi = 0;
    for (int g = 0; g < grid; ++g) {
        awq_ratio_scales(a, b, (double)g / (double)grid, s.data());
        parallel_rows(n, [&](int64_t lo, int64_t hi) {
            for (int64_t r = lo; r < hi; ++r)
                for (int64_t j = 0; j < k; ++j)
                    ws[(size_t)(r * k + j)] = w[r * k + j] * s[(size_t)j];
        });
        if (int rc = ql_awq_pack(ws.data(), n, k, group, qw.data(), sc.data(), qz.data()))
            return rc;
        for (int64_t i = 0; i < t; ++i)
            for (int64_t j = 0; j < k; ++j)
                xs[(size_t)(i * k + j)] = float_to_half_rne(xf[(size_t)(i * k + j)] / s[(size_t)j]);
        if (int rc = awq_hip(hipMemcpyAsync(dws + L.x, xs.data(), xs.size() * 2, hipMemcpyHostToDevice, st), "copy x"))
            return rc;
        if (int rc = awq_hip(hipMemcpyAsync(dws + L.qw, qw.data(), qw.size() * 4, hipMemcpyHostToDevice, st),
                             "copy qweight"))
            return rc;
        if (int rc = awq_hip(hipMemcpyAsync(dws + L.sc, sc.data(), sc.size() * 2, hipMemcpyHostToDevice, st),
                             "copy scales"))
            return rc;
        if (int rc = awq_hip(hipMemcpyAsync(dws + L.qz, qz.data(), qz.size() * 4, hipMemcpyHostToDevice, st),
                             "copy qzeros"))
            return rc;
        if (int rc = ql_w4a16_gemm(reinterpret_cast<const uint16_t*>(dws + L.x),
                                   reinterpret_cast<const int32_t*>(dws + L.qw),
                                   reinterpret_cast<const uint16_t*>(dws + L.sc),
                                   reinterpret_cast<const int32_t*>(dws + L.qz), reinterpret_cast<uint16_t*>(dws + L.y),
                                   t, n, k, group, L.ws_bytes ? dws + L.ws : nullptr, L.ws_bytes, stream))
            return rc;
        if (int rc = awq_hip(hipMemcpyAsync(y.data(), dws + L.y, y.size() * 2, hipMemcpyDeviceToHost, st), "copy y"))
            return rc;
        if (int rc = awq_hip(hipStreamSynchronize(st), "synchronise"))
            return rc;
        double e2 = 0.0;
        for (size_t e = 0; e < y.size(); ++e) {
            const double d = (double)half_to_float(y[e]) - yref[e];
            e2 += d * d;
        }
        err[g] = e2;
        if (e2 < err[bi])
            bi = g;
    }

    // 3. the chosen ratio: its smoothing vector and, if asked, its packed weights
    *best = bi;
    awq_ratio_scales(a, b, (double)bi / (double)grid, s_best);
    if (qweight || scales || qzeros) {
        if (!qweight || !scales || !qzeros)
            QL_FAIL(QL_ERR_NULL, "%s: qweight, scales and qzeros are all given or all null", who);
        parallel_rows(n, [&](int64_t lo, int64_t hi) {
            for (int64_t r = lo; r < hi; ++r)
                for (int64_t j = 0; j < k; ++j)
                    ws[(size_t)(r * k + j)] = w[r * k + j] * s_best[j];
        });
        return ql_awq_pack(ws.data(), n, k, group, qweight, scales, qzeros);
    }
    return QL_OK;
}
