// W8A8 (SmoothQuant) kernels for gfx950 and their C-ABI entry points.
//
//   quant_rmsnorm_kernel -- QRMSNorm: RMSNorm fused with per-token dynamic int8
//                           quantisation (LMDeploy W8A8 guide, "inference
//                           kernels": rms_norm_dynamic_quant, scale = absmax/127)
//   w8a8_gemm_kernel     -- int8 x int8 -> int32 MFMA GEMM with the per-token x
//                           per-channel scale epilogue (same page:
//                           matmul_kernel_dynamic_quant, c * rms_scale *
//                           linear_scale)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "ql_common.hpp"

namespace {

typedef int i4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// QRMSNorm
//
// The mean of squares is computed exactly: an fp16 value is an integer
// significand times 2^(e-25), so its square is an integer multiple of 2^-48
// below 2^80.  Each thread sums its squares in a 128-bit integer; integer
// addition is associative, so the workgroup total does not depend on the
// reduction order.  The total is divided by k and rounded once to fp32.
// Every later step (sqrt, divisions, products) is a single correctly rounded
// fp32 operation, so the codes are independent of the launch configuration.
// ---------------------------------------------------------------------------
struct U128 {
    uint64_t lo, hi;
};

__device__ __forceinline__ void add128(U128& a, uint64_t lo, uint64_t hi)
{
    a.lo += lo;
    a.hi += hi + (a.lo < lo ? 1u : 0u);
}

// square of one fp16 value, in units of 2^-48, added to acc
__device__ __forceinline__ void add_square(U128& acc, uint32_t h)
{
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t sig = h & 0x3FFu;
    if (e == 0)
        e = 1;
    else
        sig |= 0x400u;
    const uint64_t sq = (uint64_t)(sig * sig);          // < 2^22
    const uint32_t sh = 2 * e - 2;                      // 0 .. 58
    const uint64_t lo = sq << sh;
    const uint64_t hi = sh > 42 ? (sq >> (64 - sh)) : 0;
    add128(acc, lo, hi);
}

__device__ __forceinline__ int clz128_bits(const U128& v)  // bit length
{
    return v.hi ? 128 - __clzll(v.hi) : (v.lo ? 64 - __clzll(v.lo) : 0);
}

// (v * 2^-48) / k rounded to the nearest fp32, ties to even; k < 2^31.
__device__ float mean_from_exact(U128 v, uint32_t k)
{
    const int L = clz128_bits(v);
    if (L == 0)
        return 0.0f;
    // 64-bit window of v with its top bit at bit 63; d = weight of the window's lsb
    uint64_t a;
    bool rest = false;
    int d;
    if (L > 64) {
        const int sh = L - 64;   // 1 .. 63 (v < 2^127)
        a = (v.hi << (64 - sh)) | (v.lo >> sh);
        rest = (v.lo & ((1ull << sh) - 1)) != 0;
        d = sh;
    } else {
        const int sh = 64 - L;
        a = sh ? (v.lo << sh) : v.lo;
        d = -sh;
    }
    const uint64_t q1 = a / k;
    const uint64_t r1 = a - q1 * k;
    const int lq = 64 - __clzll(q1);                       // >= 33 bits since a >= 2^63
    const int drop = lq - 24;
    uint64_t mant = q1 >> drop;
    const uint64_t round = (q1 >> (drop - 1)) & 1u;
    const bool sticky = (q1 & ((1ull << (drop - 1)) - 1)) != 0 || r1 != 0 || rest;
    if (round && (sticky || (mant & 1u)))
        ++mant;
    return ldexpf((float)mant, drop + d - 48);
}

// Correctly rounded square root of a non-negative finite float.  The hardware
// estimate is within an ulp or so; it is then moved to the float whose
// rounding interval contains sqrt(x).  The boundary between two neighbouring
// floats c < c' is their midpoint m, which has at most 25 significant bits, so
// m*m is exact in fp64 and "sqrt(x) < m" is decided exactly by "x < m*m".
// (sqrt(x) never equals such a midpoint for a float x.)
__device__ float sqrt_rn(float x)
{
    if (!(x > 0.0f))
        return x == 0.0f ? x : __builtin_nanf("");
    float c = sqrtf(x);
    const double xd = (double)x;
#pragma unroll 1
    for (int it = 0; it < 4; ++it) {
        const float lo = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c) - 1u);
        const float hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c) + 1u);
        const double mlo = 0.5 * ((double)c + (double)lo);
        const double mhi = 0.5 * ((double)c + (double)hi);
        if (xd < mlo * mlo)
            c = lo;
        else if (xd > mhi * mhi)
            c = hi;
        else
            break;
    }
    return c;
}

template <int NT>
__device__ __forceinline__ U128 block_sum128(U128 v, U128* sh)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t lo = __shfl_xor(v.lo, off, 64);
        const uint64_t hi = __shfl_xor(v.hi, off, 64);
        add128(v, lo, hi);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    U128 t{0, 0};
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        add128(t, sh[w].lo, sh[w].hi);
    return t;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        t = fmaxf(t, sh[w]);
    return t;
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

constexpr int kNormThreads = 256;

// One workgroup per token; chunks of 8 fp16 (16 bytes) strided over threads.
__global__ __launch_bounds__(kNormThreads) void quant_rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ gamma, float eps,
                                                                     int8_t* __restrict__ xq,
                                                                     float* __restrict__ x_scale, int K)
{
    __shared__ U128 s_sum[kNormThreads / 64];
    __shared__ float s_max[kNormThreads / 64];
    const int row = blockIdx.x;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * K);
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    const int nch = K >> 3;

    U128 acc{0, 0};
    for (int c = threadIdx.x; c < nch; c += kNormThreads) {
        const uint4 v = xr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            add_square(acc, w[i] & 0xFFFFu);
            add_square(acc, w[i] >> 16);
        }
    }
    const U128 tot = block_sum128<kNormThreads>(acc, s_sum);
    const float ms = mean_from_exact(tot, (uint32_t)K);
    const float r = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, eps)));

    float amax = 0.0f;
    for (int c = threadIdx.x; c < nch; c += kNormThreads) {
        const uint4 v = xr[c], g = gr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y0 = __fmul_rn(__fmul_rn(h2f(w[i] & 0xFFFFu), r), h2f(gw[i] & 0xFFFFu));
            const float y1 = __fmul_rn(__fmul_rn(h2f(w[i] >> 16), r), h2f(gw[i] >> 16));
            amax = fmaxf(amax, fmaxf(fabsf(y0), fabsf(y1)));
        }
    }
    amax = block_max<kNormThreads>(amax, s_max);
    const float scale = __fdiv_rn(amax, 127.0f);
    if (threadIdx.x == 0)
        x_scale[row] = scale;

    uint2* qr = reinterpret_cast<uint2*>(xq + (int64_t)row * K);
    for (int c = threadIdx.x; c < nch; c += kNormThreads) {
        const uint4 v = xr[c], g = gr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint32_t xb = hh ? (w[i] >> 16) : (w[i] & 0xFFFFu);
                const uint32_t gb = hh ? (gw[i] >> 16) : (gw[i] & 0xFFFFu);
                const float yv = __fmul_rn(__fmul_rn(h2f(xb), r), h2f(gb));
                int qv = 0;
                if (scale > 0.0f)
                    qv = (int)rintf(__fdiv_rn(yv, scale));
                qv = qv < -127 ? -127 : (qv > 127 ? 127 : qv);
                const int e = 2 * i + hh;
                packed[e >> 2] |= ((uint32_t)qv & 0xFFu) << (8 * (e & 3));
            }
        }
        qr[c] = make_uint2(packed[0], packed[1]);
    }
}

// ---------------------------------------------------------------------------
// int8 GEMM: block tile 128 x 128, BK = 128, 4 waves as 2 x 2 (64 x 64 each),
// MFMA i32 16x16x64 i8.  Lane l supplies A[l%16][16(l/16) .. +15] and
// B[16(l/16) .. +15][l%16] (row l%16 of wq) and receives D[4(l/16)+r][l%16].
// ---------------------------------------------------------------------------
constexpr int kQBM = 128, kQBN = 128, kQBK = 128;

__device__ __forceinline__ i4_t mfma_i8(i4_t a, i4_t b, i4_t c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <bool kRaw>
__global__ __launch_bounds__(256) void w8a8_gemm_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ xs,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ ws, void* __restrict__ out,
                                                        int M, int N, int K)
{
    constexpr int CH = kQBK / 16;        // 16-byte chunks per row per step
    constexpr int RS = CH + 1;           // padded row stride (uint4)
    __shared__ uint4 at[kQBM * RS];
    __shared__ uint4 bt[kQBN * RS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, r16 = lane & 15;
    const int m0 = blockIdx.y * kQBM, n0 = blockIdx.x * kQBN;

    i4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = i4_t{0, 0, 0, 0};

    for (int kb = 0; kb < K; kb += kQBK) {
        const int nch = min(CH, (K - kb) >> 4);
        __syncthreads();
        for (int idx = threadIdx.x; idx < kQBM * CH; idx += 256) {
            const int r = idx / CH, c = idx - r * CH;
            const int m = m0 + r, n = n0 + r;
            uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && c < nch)
                va = *reinterpret_cast<const uint4*>(xq + (int64_t)m * K + kb + 16 * c);
            if (n < N && c < nch)
                vb = *reinterpret_cast<const uint4*>(wq + (int64_t)n * K + kb + 16 * c);
            at[r * RS + c] = va;
            bt[r * RS + c] = vb;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kQBK / 64; ++s) {
            const int c = 4 * s + q;
            i4_t af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = __builtin_bit_cast(i4_t, at[(wm * 64 + i * 16 + r16) * RS + c]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = __builtin_bit_cast(i4_t, bt[(wn * 64 + j * 16 + r16) * RS + c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma_i8(af[i], bf[j], acc[i][j]);
        }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + r16;
        if (n >= N)
            continue;
        const float wsn = kRaw ? 0.0f : ws[n];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + 4 * q + r;
                if (m >= M)
                    continue;
                if (kRaw) {
                    static_cast<int32_t*>(out)[(int64_t)m * N + n] = acc[i][j][r];
                } else {
                    const float v = __fmul_rn(__fmul_rn((float)acc[i][j][r], xs[m]), wsn);
                    static_cast<uint16_t*>(out)[(int64_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
                }
            }
    }
}

int launch_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        QL_FAIL(QL_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return QL_OK;
}

int check_gemm(const void* xq, const void* wq, const void* out, int64_t m, int64_t n, int64_t k, const char* who)
{
    if (m < 0 || n < 0 || k <= 0 || k % 16)
        QL_FAIL(QL_ERR_SHAPE, "%s: m=%lld n=%lld k=%lld (k must be a positive multiple of 16)", who, (long long)m,
                (long long)n, (long long)k);
    if (k > 131072 || m > (1LL << 30) || n > (1LL << 30))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: k=%lld exceeds the int32 accumulator bound (131072)", who, (long long)k);
    if (m == 0 || n == 0)
        return QL_OK;
    if (!xq || !wq || !out)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(xq) || !ql::aligned16(wq) || !ql::aligned16(out))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    return QL_OK;
}

}  // namespace

extern "C" int ql_w8a8_quant_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int8_t* xq,
                                     float* x_scale, int64_t m, int64_t k, void* stream)
{
    ql::clear_error();
    const char* who = "ql_w8a8_quant_rmsnorm";
    if (m < 0 || k <= 0 || k % 8)
        QL_FAIL(QL_ERR_SHAPE, "%s: m=%lld k=%lld (k must be a positive multiple of 8)", who, (long long)m,
                (long long)k);
    if (k > 65536 || m > (1LL << 31) - 1)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: k=%lld above 65536", who, (long long)k);
    if (!(eps >= 0.0f) || !(eps < 1e30f))
        QL_FAIL(QL_ERR_VALUE, "%s: eps must be finite and >= 0", who);
    if (m == 0)
        return QL_OK;
    if (!x || !gamma || !xq || !x_scale)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x) || !ql::aligned16(gamma) || !ql::aligned16(xq) || !ql::aligned16(x_scale))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    hipLaunchKernelGGL(quant_rmsnorm_kernel, dim3((unsigned)m), dim3(kNormThreads), 0,
                       static_cast<hipStream_t>(stream), x, gamma, eps, xq, x_scale, (int)k);
    return launch_status(who);
}

extern "C" int ql_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                            uint16_t* y, int64_t m, int64_t n, int64_t k, void* stream)
{
    ql::clear_error();
    const char* who = "ql_w8a8_gemm";
    if (int rc = check_gemm(xq, wq, y, m, n, k, who))
        return rc;
    if (m == 0 || n == 0)
        return QL_OK;
    if (!x_scale || !w_scale)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x_scale) || !ql::aligned16(w_scale))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    dim3 grid((unsigned)((n + kQBN - 1) / kQBN), (unsigned)((m + kQBM - 1) / kQBM));
    hipLaunchKernelGGL(w8a8_gemm_kernel<false>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), xq, x_scale,
                       wq, w_scale, (void*)y, (int)m, (int)n, (int)k);
    return launch_status(who);
}

extern "C" int ql_w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t m, int64_t n, int64_t k,
                                void* stream)
{
    ql::clear_error();
    const char* who = "ql_w8a8_gemm_i32";
    if (int rc = check_gemm(xq, wq, acc, m, n, k, who))
        return rc;
    if (m == 0 || n == 0)
        return QL_OK;
    dim3 grid((unsigned)((n + kQBN - 1) / kQBN), (unsigned)((m + kQBM - 1) / kQBM));
    hipLaunchKernelGGL(w8a8_gemm_kernel<true>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), xq, nullptr,
                       wq, nullptr, (void*)acc, (int)m, (int)n, (int)k);
    return launch_status(who);
}
