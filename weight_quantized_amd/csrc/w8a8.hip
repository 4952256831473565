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
#include <type_traits>

#include "lds_dma.hpp"
#include "ql_common.hpp"

namespace {

typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// QRMSNorm
//
// The mean of squares is the exact mean rounded once to fp32.  Fast path: the
// squares of fp16 values are exact in fp64 and are summed in fp64; with the
// sum's error bound, the fp32 rounding of the mean is certain unless it lies
// within 2^-36 of a rounding boundary.  Exact path (then): an fp16 value is an
// integer significand times 2^(e-25), so its square is an integer multiple of
// 2^-48 below 2^80; each thread sums its squares in a 128-bit integer
// (associative, so independent of the reduction order) and the total is
// divided by k and rounded once.  Every later step (sqrt, divisions, products)
// is a single correctly rounded fp32 operation, so the codes do not depend on
// the launch configuration.
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

// Wave reductions by DPP moves, which stay in the VALU (a shuffle is an LDS
// round trip per step): within each row of 16 lanes the quad swaps (lane ^ 1,
// lane ^ 2), the half-row mirror (lane 7 - i of each 8) and the row mirror
// (lane 15 - i) leave every lane with its row's result; the four rows are
// then combined through readlane, so every lane gets the wave's result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    // every lane enabled and every source lane within its row: the old value
    // is never used, and bound_ctrl lets the compiler leave it unset
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = dpp<CTRL>((uint32_t)b), hi = dpp<CTRL>((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, lo | (hi << 32));
}
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(uint32_t, v))));
    v = fmaxf(v, __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(uint32_t, v))));
    const auto rl = [&](int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
    };
    return fmaxf(fmaxf(rl(0), rl(16)), fmaxf(rl(32), rl(48)));
}
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh)
{
    v = wave_max(v);
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

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* sh)
{
    v = wave_sum_f64(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        t += sh[w];
    return t;
}

// Fast path of the mean of squares.  `tot` is the sum of K exact fp64
// squares (non-negative) accumulated with K + log2(NT) roundings at most, so
// |tot - exact| <= 2^-37 exact for K <= 65536; dividing by K adds one more
// rounding.  If no fp32 rounding boundary (the midpoint to either neighbour of
// the candidate, exact in fp64) lies within 2^-36 of tot / K, the candidate is
// the correctly rounded exact mean; otherwise the caller takes the exact path.
__device__ __forceinline__ bool mean_fast(double tot, int K, float* out)
{
    const double m = tot / (double)K;
    if (m == 0.0) {
        *out = 0.0f;
        return true;
    }
    const float f = (float)m;
    const uint32_t fb = __builtin_bit_cast(uint32_t, f);
    const double lo = 0.5 * ((double)f + (double)__builtin_bit_cast(float, fb - 1u));
    const double hi = 0.5 * ((double)f + (double)__builtin_bit_cast(float, fb + 1u));
    const double d = m * 0x1p-36;
    *out = f;
    return m - d > lo && m + d < hi;
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

// a * b rounded once to fp32, signed zeros kept, with one of the operands an
// fp16 half of a 32-bit word (HI: bits 16-31): v_fma_mix_f32 with the addend
// -0 (the exact product plus -0 is the exact product, whatever its sign).  The
// compiler turns fma(a, b, -0) back into a conversion and a multiply.
template <bool HI>
__device__ __forceinline__ float mul_hf(uint32_t w, float b, float negzero)
{
    float d;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(b), "v"(negzero));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(b), "v"(negzero));
    return d;
}

constexpr int kNormThreads = 256;

// One workgroup per token; chunks of 8 fp16 (16 bytes) strided over threads.
// CPT > 0: each thread holds its CPT chunks of x and gamma in registers --
// every load of the token is issued before the first is used, and the norm,
// absmax and quantisation passes read registers.  CPT == 0: chunks are
// re-read from memory in each pass (any k).  Chunks past k are zero: they add
// nothing to the sum of squares or the absmax and are not stored.
// Eight fp16 pairs -> fp16(a + b) per element: the correctly rounded binary16
// sum, which is also the fp32 sum rounded to binary16 (24 >= 2 * 11 + 2
// significand bits, so the double rounding is innocuous).
__device__ __forceinline__ uint4 add_h8(uint4 a, uint4 b)
{
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)   // one v_pk_add_f16 per pair
        o[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, aw[e]) + __builtin_bit_cast(h2v, bw[e]));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Per-token quantisers, one workgroup per token.  MODE:
//   kNormQuant    -- QRMSNorm: y = RMSNorm(x) * gamma, then per-token int8
//   kAddNormQuant -- h = fp16(x + residual) written to h_out (the residual
//                    stream; h_out may be residual itself), then QRMSNorm of h
//   kTokenQuant   -- y = x (no norm, no gamma), then per-token int8
//   kNormQuantF8, kTokenQuantF8 -- as kNormQuant and kTokenQuant with FP8
//                    E4M3 codes: x_scale = max|y| / 448, code = e4m3(y / x_scale)
// x, residual and h_out are not restrict: h_out may be x or residual, and an
// in-place update reads each chunk before the same thread overwrites it.
constexpr int kNormQuant = 0, kAddNormQuant = 1, kTokenQuant = 2, kNormQuantF8 = 3, kTokenQuantF8 = 4;

template <int CPT, int MODE, int NT = kNormThreads>
__global__ __launch_bounds__(NT) void quant_rmsnorm_kernel(const uint16_t* x,
                                                                     const uint16_t* residual,
                                                                     const uint16_t* __restrict__ gamma, float eps,
                                                                     uint16_t* h_out, int8_t* __restrict__ xq,
                                                                     float* __restrict__ x_scale, int K)
{
    constexpr bool kF8 = MODE == kNormQuantF8 || MODE == kTokenQuantF8;
    constexpr bool kNoNorm = MODE == kTokenQuant || MODE == kTokenQuantF8;
    __shared__ U128 s_sum[NT / 64];
    __shared__ double s_sumd[NT / 64];
    __shared__ float s_max[NT / 64];
    const int row = blockIdx.x;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * K);
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    const int nch = K >> 3;
    constexpr int R = CPT > 0 ? CPT : 1;
    uint4 xv[R], gv[R];
    if constexpr (MODE == kAddNormQuant && CPT == 0) {
        // chunks are re-read in every pass: form h once, then read it back
        // (each thread reads only the chunks it wrote)
        const uint4* rr = reinterpret_cast<const uint4*>(residual + (int64_t)row * K);
        uint4* hr = reinterpret_cast<uint4*>(h_out + (int64_t)row * K);
        for (int c = (int)threadIdx.x; c < nch; c += NT)
            hr[c] = add_h8(xr[c], rr[c]);
        xr = hr;
    }
    auto chunk = [&](int i, int c, uint4& v, uint4& g) {   // chunk c (loop slot i)
        if constexpr (CPT > 0) {
            v = xv[i];
            g = gv[i];
        } else {
            v = xr[c];
            g = kNoNorm ? make_uint4(0u, 0u, 0u, 0u) : gr[c];
        }
    };
    if constexpr (CPT > 0) {
        uint4 rv[MODE == kAddNormQuant ? CPT : 1];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = (int)threadIdx.x + i * NT;
            const int cc = c < nch ? c : nch - 1;
            xv[i] = xr[cc];
            gv[i] = kNoNorm ? make_uint4(0u, 0u, 0u, 0u) : gr[cc];
            if constexpr (MODE == kAddNormQuant)
                rv[i] = reinterpret_cast<const uint4*>(residual + (int64_t)row * K)[cc];
        }
        if constexpr (MODE == kAddNormQuant) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = (int)threadIdx.x + i * NT;
                xv[i] = add_h8(xv[i], rv[i]);
                if (c < nch)
                    reinterpret_cast<uint4*>(h_out + (int64_t)row * K)[c] = xv[i];
            }
        }
        if (nch < CPT * NT) {   // a uniform test: only a ragged k has chunks past its end
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                if ((int)threadIdx.x + i * NT >= nch)
                    xv[i] = gv[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const int npass = CPT > 0 ? CPT : (nch - (int)threadIdx.x + NT - 1) / NT;

    // mean of squares: fp64 sum of the exact squares, or, when its fp32
    // rounding is not certain, the exact 128-bit integer sum (the decision is
    // taken on the workgroup total, so the whole workgroup branches together)
    float r = 1.0f;
    if constexpr (!kNoNorm) {
        double accd = 0.0;
#pragma unroll R
        for (int i = 0; i < npass; ++i) {
            uint4 v, g;
            chunk(i, (int)threadIdx.x + i * NT, v, g);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double a = (double)h2f(w[e] & 0xFFFFu), b = (double)h2f(w[e] >> 16);
                accd = __builtin_fma(a, a, accd);
                accd = __builtin_fma(b, b, accd);
            }
        }
        float ms;
        if (!mean_fast(block_sum_f64<NT>(accd, s_sumd), K, &ms)) {
            U128 acc{0, 0};
#pragma unroll R
            for (int i = 0; i < npass; ++i) {
                uint4 v, g;
                chunk(i, (int)threadIdx.x + i * NT, v, g);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    add_square(acc, w[e] & 0xFFFFu);
                    add_square(acc, w[e] >> 16);
                }
            }
            ms = mean_from_exact(block_sum128<NT>(acc, s_sum), (uint32_t)K);
        }
        r = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, eps)));
    }

    // y = fp32(fp32(x * r) * gamma) (y = x without the norm); kept per
    // element when the chunks are in registers, recomputed per pass otherwise
    float yk[R][8];
    const float nz = -0.0f;
    auto y_of = [&](const uint4& v, const uint4& g, float (&yo)[8]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (kNoNorm) {
                yo[2 * e] = h2f(w[e] & 0xFFFFu);
                yo[2 * e + 1] = h2f(w[e] >> 16);
            } else {
                // each product rounded once, fp16 operands converted inside
                // the instruction (the e4m3 codes keep the sign of a zero)
                yo[2 * e] = mul_hf<false>(gw[e], mul_hf<false>(w[e], r, nz), nz);
                yo[2 * e + 1] = mul_hf<true>(gw[e], mul_hf<true>(w[e], r, nz), nz);
            }
        }
    };
    float amax = 0.0f;
#pragma unroll R
    for (int i = 0; i < npass; ++i) {
        uint4 v, g;
        chunk(i, (int)threadIdx.x + i * NT, v, g);
        float yo[8];
        y_of(v, g, yo);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            amax = fmaxf(amax, fabsf(yo[e]));
            if constexpr (CPT > 0)
                yk[i][e] = yo[e];
        }
    }
    amax = block_max<NT>(amax, s_max);
    const float scale = __fdiv_rn(amax, kF8 ? 448.0f : 127.0f);
    if (threadIdx.x == 0)
        x_scale[row] = scale;

    // Codes of y: rint(fp32(y / scale)), clamped to +-127.  q0 = y *
    // RN(1/scale) is within 1.5 ulp of fp32(y / scale) (both < 128 in
    // magnitude, an ulp is at most 2^-17), so the two round to the same integer
    // unless q0 lies within 2^-15 of a half-integer, i.e. unless q0 - rint(q0)
    // (exact) is at least 1/2 - 2^-15 in magnitude; only those take the exact
    // division.  Eight codes at a time, packed four to a word by byte permutes.
    const float rcp = scale > 0.0f ? __fdiv_rn(1.0f, scale) : 0.0f;
    auto codes8 = [&](const float (&yv)[8], uint32_t (&pk)[2]) {
        if (!(scale > 0.0f)) {
            pk[0] = pk[1] = 0u;
            return;
        }
        float qf[8];
        bool near = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q0 = yv[e] * rcp;
            qf[e] = rintf(q0);
            near |= fabsf(q0 - qf[e]) >= 0.5f - 0x1p-15f;
        }
        if (__builtin_expect(near, 0)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float q0 = yv[e] * rcp;
                if (fabsf(q0 - qf[e]) >= 0.5f - 0x1p-15f)
                    qf[e] = rintf(__fdiv_rn(yv[e], scale));
            }
        }
        // No clamp to +-127 is needed: scale > 0 implies every y is finite
        // (a NaN or infinite element leaves max|y| = 0, hence scale = 0), and
        // with scale = RN(max|y| / 127) >= (max|y| / 127) / (1 + 2^-24), both
        // |y / scale| and |y * RN(1 / scale)| are below 127 (1 + 2^-24)^3 <
        // 127.5 before their own rounding, so every code rounds to at most 127.
        uint32_t qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qv[e] = (uint32_t)(int)qf[e];
        // byte 0 of each code: perm selector bytes 0 / 4 pick the low byte of
        // the second / first operand, 0x0C a zero byte
#pragma unroll
        for (int h = 0; h < 2; ++h)
            pk[h] = __builtin_amdgcn_perm(qv[4 * h + 1], qv[4 * h], 0x0C0C0400u) |
                    __builtin_amdgcn_perm(qv[4 * h + 3], qv[4 * h + 2], 0x04000C0Cu);
    };
    // FP8 codes of eight y: e4m3(fp32(y / scale)), 0 for a zero scale.  q0 = y
    // * RN(1/scale) differs from fp32(y / scale) by less than 3 * 2^-24 of its
    // magnitude, fewer than 8 fp32 steps either way.  The cast is monotone and
    // rounds q and -q alike, so when |q0| eight steps down and eight steps up
    // cast to the same code, so does fp32(y / scale), and q0 gives the code;
    // otherwise (rare) that quotient is formed by the correctly rounded
    // division.  Casts take two values per instruction (nearest, ties to even;
    // no quotient exceeds 448 by more than rounding).
    auto cvt4 = [](float a, float b, float c, float d) -> uint32_t {
        const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
    };
    auto codes_f8 = [&](const float (&yv)[8], uint32_t (&pk)[2]) {
        if (!(scale > 0.0f)) {
            pk[0] = pk[1] = 0u;
            return;
        }
        float qf[8], lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qf[e] = yv[e] * rcp;
            const uint32_t a = __builtin_bit_cast(uint32_t, qf[e]) & 0x7FFFFFFFu;
            lo[e] = __builtin_bit_cast(float, __builtin_elementwise_sub_sat(a, 8u));
            hi[e] = __builtin_bit_cast(float, a + 8u);
        }
        uint32_t dif[2];
        bool near = false;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            dif[h] = cvt4(lo[4 * h], lo[4 * h + 1], lo[4 * h + 2], lo[4 * h + 3]) ^
                     cvt4(hi[4 * h], hi[4 * h + 1], hi[4 * h + 2], hi[4 * h + 3]);
            near |= dif[h] != 0u;
        }
        if (__builtin_expect(near, 0)) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((dif[e >> 2] >> (8 * (e & 3))) & 0xFFu)
                    qf[e] = __fdiv_rn(yv[e], scale);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            pk[h] = cvt4(qf[4 * h], qf[4 * h + 1], qf[4 * h + 2], qf[4 * h + 3]);
    };
    uint2* qr = reinterpret_cast<uint2*>(xq + (int64_t)row * K);
#pragma unroll R
    for (int i = 0; i < npass; ++i) {
        const int c = (int)threadIdx.x + i * NT;
        float yo[8];
        if constexpr (CPT > 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                yo[e] = yk[i][e];
        } else {
            uint4 v, g;
            chunk(i, c, v, g);
            y_of(v, g, yo);
        }
        uint32_t packed[2] = {0u, 0u};
        if constexpr (kF8)
            codes_f8(yo, packed);
        else
            codes8(yo, packed);
        if (c < nch)
            qr[c] = make_uint2(packed[0], packed[1]);
    }
}

// ---------------------------------------------------------------------------
// int8 GEMM.  Block tile BM x BN, K advanced in tiles of 128 bytes, 4 waves as
// 2 x 2 (wave tile BM/2 x BN/2), MFMA i32 16x16x64 i8.  Lane l supplies
// A[l%16][16(l/16) .. +15] and B[16(l/16) .. +15][l%16] (row l%16 of wq) and
// receives D[4(l/16)+r][l%16].
//
// Both operands are K-major, so a k-tile of either is BM (BN) rows of 128
// contiguous bytes: every global load fetches whole 128-byte lines.  Tiles are
// double-buffered in LDS; the next k-tile is fetched into registers while the
// current one is multiplied, then written to the other buffer.  LDS rows are
// padded to 144 bytes so the 16 rows of an MFMA fragment read fall in
// distinct banks.
//
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2); the tile order below gives every XCD a contiguous run of tiles that
// sweeps N for one M block, so that block of A stays in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kQBK = 128;                 // k bytes per tile
constexpr int kQRow = kQBK + 16;          // padded LDS row (bytes)
constexpr int kXcds = 8;

__device__ __forceinline__ i4_t mfma_i8(i4_t a, i4_t b, i4_t c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// MFMA 32x32x32 int8 -> int32.  Lane l supplies A[l%32][16(l/32) .. +15] and
// B[16(l/32) .. +15][l%32]; it receives D[8(v/4) + 4(l/32) + v%4][l%32] in
// element v, v = 0..15.  At one wave per SIMD it sustains over 90% of the
// int8 peak, against under 60% for the 16x16x64 form.
__device__ __forceinline__ i16_t mfma_i8_32(i4_t a, i4_t b, i16_t c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// FP8 E4M3 x E4M3 -> fp32, MFMA 32x32x64 (format code 0 = E4M3 for both
// operands, unit E8M0 block scales 127 = 2^0).  A lane's 32 codes are the two
// 16-byte fragments of consecutive 32-byte k-steps; A and B are built alike,
// so the instruction covers the 64 k once, in some order of k.
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef int i8v_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16v_t mfma_f8_64(i8v_t a, i8v_t b, f16v_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ float acc_f(int v) { return (float)v; }
__device__ __forceinline__ float acc_f(float v) { return v; }

// tile index of workgroup `wg` so that each XCD gets a contiguous run of tiles
__device__ __forceinline__ int xcd_tile(int wg, int ntiles)
{
    const int per = (ntiles + kXcds - 1) / kXcds;
    const int t = (wg % kXcds) * per + wg / kXcds;
    return t;
}

// One output of the fp16 epilogue: y = fp16(fp32(fp32(acc * x_scale) *
// w_scale) [+ bias] [+ residual]), every operation rounded to fp32 on its own
// (the build does not contract), the bias and residual terms only when given,
// then one rounding to fp16 (the empty asm keeps the conversion from being
// fused with the last operation).
struct EpiTerms {
    const uint16_t* bias;   // [N] fp16 or null
    const uint16_t* res;    // [M, N] fp16 or null; may be the output itself
};
__device__ __forceinline__ uint32_t epi_h(float acc, float xs, float ws, const EpiTerms& et, float b, float r)
{
    float f = __fmul_rn(__fmul_rn(acc, xs), ws);
    if (et.bias)
        f = __fadd_rn(f, b);
    if (et.res)
        f = __fadd_rn(f, r);
    asm volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float h_lo(uint32_t w) { return h2f(w & 0xFFFFu); }
__device__ __forceinline__ float h_hi(uint32_t w) { return h2f(w >> 16); }

// Epilogue of both int8 GEMM kernels.  The MFMA takes the weight fragment as
// its A operand and the activation fragment as B, so fragment (i, j) holds the
// transposed product: lane (q, r16) has y[m][n .. n+3] with m = mrow + 16 i,
// n = ncol + 16 j, mrow = tile row of r16, ncol = tile column 4 q, i.e. four
// consecutive outputs of one row (one 8-byte fp16 or 16-byte int32 store).
// Every scale is loaded first at a clamped index so the loads are in flight
// together.  `vec`: the whole tile is in bounds and rows are 4-aligned.
template <int FI, int FJ, bool kRaw>
__device__ __forceinline__ void store_tile(const i4_t (&acc)[FI][FJ], const float* __restrict__ xs,
                                           const float* __restrict__ ws, const EpiTerms& et, void* out, int M,
                                           int N, int mrow, int ncol, bool vec)
{
    float xsv[FI], wsv[FJ][4], bsv[FJ][4];
    if (!kRaw) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
            xsv[i] = xs[min(mrow + 16 * i, M - 1)];
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wsv[j][r] = ws[min(ncol + 16 * j + r, N - 1)];
                bsv[j][r] = et.bias ? h2f(et.bias[min(ncol + 16 * j + r, N - 1)]) : 0.0f;
            }
    }
    auto to_h = [&](int i, int j, int r, float rv) -> uint32_t {
        return epi_h((float)acc[i][j][r], xsv[i], wsv[j][r], et, bsv[j][r], rv);
    };
    if (vec) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int64_t o = (int64_t)(mrow + 16 * i) * N + ncol + 16 * j;
                if (kRaw) {
                    *reinterpret_cast<i4_t*>(static_cast<int32_t*>(out) + o) = acc[i][j];
                } else {
                    const uint2 rr = et.res ? *reinterpret_cast<const uint2*>(et.res + o) : make_uint2(0u, 0u);
                    uint2 h;
                    h.x = to_h(i, j, 0, h_lo(rr.x)) | (to_h(i, j, 1, h_hi(rr.x)) << 16);
                    h.y = to_h(i, j, 2, h_lo(rr.y)) | (to_h(i, j, 3, h_hi(rr.y)) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = h;
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        const int m = mrow + 16 * i;
        if (m >= M)
            continue;
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = ncol + 16 * j + r;
                if (n >= N)
                    continue;
                const int64_t o = (int64_t)m * N + n;
                if (kRaw)
                    static_cast<int32_t*>(out)[o] = acc[i][j][r];
                else
                    static_cast<uint16_t*>(out)[o] = (uint16_t)to_h(i, j, r, et.res ? h2f(et.res[o]) : 0.0f);
            }
    }
}

// Epilogue of the pipelined kernel (32x32 MFMA tiles, weights as the A
// operand): fragment (i, j) of a wave holds y rows mrow + 32 i + l%32 and
// columns ncol + 32 j + 8 (v/4) + 4 (l/32) + v%4, so each lane owns runs of
// four consecutive columns (8-byte fp16 stores).  Same rounding as store_tile.
template <int FI, int FJ, bool kRaw, class AccT>
__device__ __forceinline__ void store_tile32(const AccT (&acc)[FI][FJ], const float* __restrict__ xs,
                                             const float* __restrict__ ws, const EpiTerms& et, void* out, int M,
                                             int N, int mrow, int ncol, bool vec)
{
    float xsv[FI], wsv[FJ][16], bsv[FJ][16];
    if (!kRaw) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
            xsv[i] = xs[min(mrow + 32 * i, M - 1)];
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int n = min(ncol + 32 * j + 8 * (v >> 2) + (v & 3), N - 1);
                wsv[j][v] = ws[n];
                bsv[j][v] = et.bias ? h2f(et.bias[n]) : 0.0f;
            }
    }
    auto to_h = [&](int i, int j, int v, float rv) -> uint32_t {
        return epi_h(acc_f(acc[i][j][v]), xsv[i], wsv[j][v], et, bsv[j][v], rv);
    };
    if (vec) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t o = (int64_t)(mrow + 32 * i) * N + ncol + 32 * j + 8 * g;
                    if constexpr (kRaw) {
                        const i4_t v4 = i4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                             acc[i][j][4 * g + 3]};
                        *reinterpret_cast<i4_t*>(static_cast<int32_t*>(out) + o) = v4;
                    } else {
                        const uint2 rr = et.res ? *reinterpret_cast<const uint2*>(et.res + o) : make_uint2(0u, 0u);
                        uint2 h;
                        h.x = to_h(i, j, 4 * g, h_lo(rr.x)) | (to_h(i, j, 4 * g + 1, h_hi(rr.x)) << 16);
                        h.y = to_h(i, j, 4 * g + 2, h_lo(rr.y)) | (to_h(i, j, 4 * g + 3, h_hi(rr.y)) << 16);
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = h;
                    }
                }
        return;
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        const int m = mrow + 32 * i;
        if (m >= M)
            continue;
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int n = ncol + 32 * j + 8 * (v >> 2) + (v & 3);
                if (n >= N)
                    continue;
                const int64_t o = (int64_t)m * N + n;
                if constexpr (kRaw)
                    static_cast<int32_t*>(out)[o] = acc[i][j][v];
                else
                    static_cast<uint16_t*>(out)[o] = (uint16_t)to_h(i, j, v, et.res ? h2f(et.res[o]) : 0.0f);
            }
    }
}

template <int BM, int BN, bool kRaw>
__global__ __launch_bounds__(256) void w8a8_gemm_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ xs,
                                                        const int8_t* __restrict__ wq,
                                                        const float* __restrict__ ws, EpiTerms et, void* out,
                                                        int M, int N, int K)
{
    constexpr int TM = BM / 2, TN = BN / 2;           // wave tile
    constexpr int FI = TM / 16, FJ = TN / 16;          // MFMA tiles per wave
    constexpr int ACH = BM * (kQBK / 16) / 256;        // A 16-byte chunks per thread per tile
    constexpr int BCH = BN * (kQBK / 16) / 256;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * kQRow];
    uint8_t* const As = lds;
    uint8_t* const Bs = lds + 2 * BM * kQRow;

    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int tile = xcd_tile(blockIdx.x, tm * tn);
    if (tile >= tm * tn)
        return;
    const int m0 = (tile / tn) * BM, n0 = (tile % tn) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, r16 = lane & 15;

    // global -> register staging of one k-tile
    uint4 ra[ACH], rb[BCH];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int u = 0; u < ACH; ++u) {
            const int c = tid + u * 256;
            const int row = c >> 3, col = (c & 7) * 16;
            const int m = m0 + row, k = kb + col;
            const bool ok = m < M && k < K;
            ra[u] = *reinterpret_cast<const uint4*>(xq + (int64_t)(ok ? m : 0) * K + (ok ? k : 0));
            if (!ok)
                ra[u] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < BCH; ++u) {
            const int c = tid + u * 256;
            const int row = c >> 3, col = (c & 7) * 16;
            const int n = n0 + row, k = kb + col;
            const bool ok = n < N && k < K;
            rb[u] = *reinterpret_cast<const uint4*>(wq + (int64_t)(ok ? n : 0) * K + (ok ? k : 0));
            if (!ok)
                rb[u] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < ACH; ++u) {
            const int c = tid + u * 256;
            *reinterpret_cast<uint4*>(As + buf * BM * kQRow + (c >> 3) * kQRow + (c & 7) * 16) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < BCH; ++u) {
            const int c = tid + u * 256;
            *reinterpret_cast<uint4*>(Bs + buf * BN * kQRow + (c >> 3) * kQRow + (c & 7) * 16) = rb[u];
        }
    };

    i4_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            acc[i][j] = i4_t{0, 0, 0, 0};

    const int nk = (K + kQBK - 1) / kQBK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            fetch((kt + 1) * kQBK);
        const uint8_t* a_base = As + buf * BM * kQRow + (wm * TM + r16) * kQRow + q * 16;
        const uint8_t* b_base = Bs + buf * BN * kQRow + (wn * TN + r16) * kQRow + q * 16;
#pragma unroll
        for (int s = 0; s < kQBK / 64; ++s) {
            i4_t af[FI], bf[FJ];
#pragma unroll
            for (int i = 0; i < FI; ++i)
                af[i] = *reinterpret_cast<const i4_t*>(a_base + i * 16 * kQRow + s * 64);
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                bf[j] = *reinterpret_cast<const i4_t*>(b_base + j * 16 * kQRow + s * 64);
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = mfma_i8(bf[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk)
            stash(buf ^ 1);
        __syncthreads();
    }

    const bool vec = m0 + BM <= M && n0 + BN <= N && (N & 3) == 0;
    store_tile<FI, FJ, kRaw>(acc, xs, ws, et, out, M, N, m0 + wm * TM + r16, n0 + wn * TN + 4 * q, vec);
}

constexpr int kQBM = 256, kQBN = 128;

// ---------------------------------------------------------------------------
// int8 GEMM, pipelined (K % BK == 0).  The same 2x2-wave MFMA tiling as above,
// but the operands go straight from global memory into a ring of S LDS stages
// with the gfx950 direct global->LDS load (16 bytes per lane; a wave's 64
// lanes fill 1 KiB of LDS contiguously), so up to S-1 k-tiles are in flight
// without holding them in registers.
//
// The loads and the stage handshake are inline assembly: the compiler does not
// track which LDS stage a direct load fills and would wait for every
// outstanding load before any LDS read, serialising the ring.  Here each wave
// waits (vmcnt) only for its own loads of the stage it needs next, then a
// barrier makes every wave's part of that stage visible.
//
// MFMA fragments are double-buffered in registers per 64-byte k-step: the LDS
// reads of step t+1 are in flight while step t is multiplied.  The barrier of
// a stage sits before its first step is read, after every wave has read the
// whole previous stage, whose slot is then refilled.
//
// LDS rows are BK bytes (BK/16 chunks of 16).  Logical chunk c of tile row r
// sits at physical chunk c ^ f(r), f = a 64-byte-row swizzle for 32-row fragments
// or the 128-byte-row one, measured free of bank conflicts for these reads.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int swz(int r)
{
    return BK == 64 ? ql::swz64x32(r) : ql::swz128(r);
}

template <int BM_, int BN_, int BK_, int S_, bool kMapN_, int NW_ = 4>
struct PipeCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr bool kMapN = kMapN_;   // tile order: m fastest (true) or n fastest
    static constexpr int NW = NW_;           // waves, 2 x NW/2 over the tile
    static constexpr int WN = NW / 2;
    static constexpr int KS = BK / 32;       // MFMA k-steps per stage
    static constexpr int CH = BK / 16;       // 16-byte chunks per LDS row
    static constexpr int RPB = 1024 / BK;    // rows filled by one 1 KiB wave load
    static constexpr int kStageBytes = (BM + BN) * BK;
    static constexpr int kLds = S * kStageBytes;
    static constexpr int D = (BM + BN) / RPB / NW;  // direct loads per wave per stage
    static constexpr int DA = BM / RPB / NW;        // ... of them activation rows
    static constexpr int kWgPerCu = kLds <= 80 * 1024 ? 2 : 1;   // workgroups that fit one CU's LDS
    static_assert(BK == 64 || BK == 128, "k-tile of 64 or 128 bytes");
    static_assert((BM + BN) % (NW * RPB) == 0 && BM % (NW * RPB) == 0,
                  "whole 1 KiB blocks, every wave's loads split alike between X and W");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(S >= 2 && D * (S - 1) < 64, "ring depth within vmcnt");
};

template <class C, bool kRaw, bool kF8 = false>
__global__ __launch_bounds__(C::NW * 64, C::kWgPerCu) void w8a8_gemm_pipe_kernel(const int8_t* __restrict__ xq,
                                                             const float* __restrict__ xs,
                                                             const int8_t* __restrict__ wq,
                                                             const float* __restrict__ ws, EpiTerms et,
                                                             void* out, int M, int N, int K)
{
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, S = C::S, KS = C::KS, D = C::D, NW = C::NW;
    constexpr int TM = BM / 2, TN = BN / C::WN;
    constexpr int FI = TM / 32, FJ = TN / 32;          // 32x32 MFMA tiles per wave
    extern __shared__ __attribute__((aligned(1024))) uint8_t pl[];   // S * kStageBytes

    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int tile = xcd_tile(blockIdx.x, tm * tn);
    if (tile >= tm * tn)
        return;
    const int m0 = (C::kMapN ? tile % tm : tile / tn) * BM;
    const int n0 = (C::kMapN ? tile / tm : tile % tn) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)pl;

    // This wave's direct loads: the stage is (BM + BN) rows of BK bytes in
    // blocks of RPB rows (1 KiB); wave w fills blocks w, w+NW, ...: its first
    // DA loads are activation rows, the rest weight rows.  Lane l of a block
    // writes physical chunk l % CH of row l / CH, i.e. it reads logical chunk
    // (l % CH) ^ f(row).  Rows past M or N re-read the last row.  Each load is
    // a wave-uniform base (the operand advanced to k-tile kt, in scalar
    // registers) plus a fixed 32-bit per-lane offset (the host sends operands
    // of 4 GiB or more to the register-staged kernel), and its LDS
    // destination is wave-uniform too, so issuing a load costs no vector
    // instruction.
    constexpr int DA = C::DA;
    uint32_t soff[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
        const int blk = wave + NW * u;
        const int row = blk * C::RPB + lane / C::CH;
        const int c = (lane % C::CH) ^ swz<BK>(row);
        if (u < DA) {
            const int m = min(m0 + row, M - 1);
            soff[u] = (uint32_t)m * (uint32_t)K + 16u * (uint32_t)c;
        } else {
            const int n = min(n0 + row - BM, N - 1);
            soff[u] = (uint32_t)n * (uint32_t)K + 16u * (uint32_t)c;
        }
    }
    const uint32_t wdst = (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)wave * 1024u);
    auto issue = [&](int kt, int slot) {
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(xq) + (int64_t)kt * BK;
        const uint8_t* wb = reinterpret_cast<const uint8_t*>(wq) + (int64_t)kt * BK;
#pragma unroll
        for (int u = 0; u < D; ++u)
            ql::dma16s(u < DA ? xb : wb, soff[u], wdst + (uint32_t)(slot * C::kStageBytes + NW * u * 1024));
    };

    using AccT = std::conditional_t<kF8, f16v_t, i16_t>;
    static_assert(!(kF8 && kRaw), "FP8 has no raw accumulator export");
    AccT acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            acc[i][j] = AccT{};

    // fragments of k-step j (32 bytes of k) of a stage: lane l reads row
    // l%32 of the fragment, chunk 2j + l/32, swizzled
    const int r32 = lane & 31, h32 = lane >> 5;
    const int arow0 = wm * TM + r32, brow0 = BM + wn * TN + r32;
    i4_t fa[2][FI], fb[2][FJ];
    auto read_frags = [&](int slot, int j, i4_t (&af)[FI], i4_t (&bf)[FJ]) {
        const uint8_t* base = pl + slot * C::kStageBytes;
        const int c = 2 * j + h32;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int r = arow0 + 32 * i;
            af[i] = *reinterpret_cast<const i4_t*>(base + r * BK + 16 * (c ^ swz<BK>(r)));
        }
#pragma unroll
        for (int jj = 0; jj < FJ; ++jj) {
            const int r = brow0 + 32 * jj;
            bf[jj] = *reinterpret_cast<const i4_t*>(base + r * BK + 16 * (c ^ swz<BK>(r)));
        }
    };

    const int nk = K / BK;
    // prologue: every slot in flight (tiles past the end reload the last one)
#pragma unroll
    for (int s = 0; s < S; ++s)
        issue(s < nk ? s : nk - 1, s);
    ql::stage_barrier<D * (S - 1)>();   // tile 0 landed

    if constexpr (kF8) {
        // FP8: one 64-k MFMA per pair of 32-byte steps.  fa8 / fb8 hold the
        // pair's two fragments (even step in the low half); after the pair's
        // MFMAs the next pair is read into the same registers (the next tile's
        // first pair after the barrier and refill).
        i8v_t fa8[FI], fb8[FJ];
        auto read_pair = [&](int slot, int j) {
            i4_t a0[FI], b0[FJ], a1[FI], b1[FJ];
            read_frags(slot, j, a0, b0);
            read_frags(slot, j + 1, a1, b1);
#pragma unroll
            for (int i = 0; i < FI; ++i)
                fa8[i] = i8v_t{a0[i][0], a0[i][1], a0[i][2], a0[i][3], a1[i][0], a1[i][1], a1[i][2], a1[i][3]};
#pragma unroll
            for (int jj = 0; jj < FJ; ++jj)
                fb8[jj] = i8v_t{b0[jj][0], b0[jj][1], b0[jj][2], b0[jj][3], b1[jj][0], b1[jj][1], b1[jj][2],
                                b1[jj][3]};
        };
        read_pair(0, 0);
        for (int kt = 0, slot = 0; kt < nk; ++kt) {
            const int next = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
            for (int j = 0; j < KS; j += 2) {
#pragma unroll
                for (int i = 0; i < FI; ++i)
#pragma unroll
                    for (int jj = 0; jj < FJ; ++jj)
                        acc[i][jj] = mfma_f8_64(fb8[jj], fa8[i], acc[i][jj]);
                __builtin_amdgcn_sched_barrier(0);
                if (j + 2 < KS) {
                    read_pair(slot, j + 2);
                } else {
                    ql::stage_barrier<D * (S - 2)>();
                    issue(kt + S < nk ? kt + S : nk - 1, slot);
                    read_pair(next, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            slot = next;
        }
    } else {
    read_frags(0, 0, fa[0], fb[0]);

    // One k-tile per iteration with its KS steps unrolled and no branch
    // inside: the last tile, too, refills its slot (with itself) and reads
    // fragments of the next slot that are never used.  A branch there would
    // join two paths, and the compiler's LDS wait before the last step's
    // MFMAs would then also cover the next tile's reads issued just before.
    static_assert(KS % 2 == 0, "register buffer index restarts with each tile");
    for (int kt = 0, slot = 0; kt < nk; ++kt) {
        const int next = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int cur = j & 1;
            if (j + 1 < KS) {
                read_frags(slot, j + 1, fa[cur ^ 1], fb[cur ^ 1]);
            } else {
                // tile kt+1 landed (S-2 younger tiles may be pending) and
                // every wave has read tile kt: refill its slot
                ql::stage_barrier<D * (S - 2)>();
                issue(kt + S < nk ? kt + S : nk - 1, slot);
                read_frags(next, 0, fa[cur ^ 1], fb[cur ^ 1]);
            }
            // keep the reads ahead of this step's MFMAs (the scheduler would
            // otherwise sink each read to its use in the next step)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int jj = 0; jj < FJ; ++jj)
                    acc[i][jj] = mfma_i8_32(fb[cur][jj], fa[cur][i], acc[i][jj]);
            __builtin_amdgcn_sched_barrier(0);
        }
        slot = next;
    }
    }
    ql::stage_barrier<0>();     // drain the trailing reloads before the workgroup exits

    const bool full = m0 + BM <= M && n0 + BN <= N;
    // Whole tile: each wave converts its TM x TN sub-tile to fp16 through its
    // own LDS area (half the rows at a time, row pitch TN + 8 halves), then
    // writes whole 16-byte chunks of whole rows, TN / 8 lanes per row, so every
    // store instruction fills complete 128-byte lines.  (The MFMA layout alone
    // would give each lane runs of 4 columns in 32 rows.)
    constexpr int PITCH = TN + 8;
    constexpr int HALF = TM / 2;
    constexpr bool kStaged = NW * HALF * PITCH * 2 <= C::kLds && FI % 2 == 0;
    if constexpr (!kRaw && kStaged) {
        if (full && (N & 7) == 0) {
            uint16_t* ot = reinterpret_cast<uint16_t*>(pl) + wave * HALF * PITCH;
            float xsv[FI], wsv[FJ][16], bsv[FJ][16];
#pragma unroll
            for (int i = 0; i < FI; ++i)
                xsv[i] = xs[m0 + wm * TM + 32 * i + r32];
#pragma unroll
            for (int jj = 0; jj < FJ; ++jj)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int n = n0 + wn * TN + 32 * jj + 8 * (v >> 2) + 4 * h32 + (v & 3);
                    wsv[jj][v] = ws[n];
                    bsv[jj][v] = et.bias ? h2f(et.bias[n]) : 0.0f;
                }
            auto to_h = [&](int i, int jj, int v, float rv) -> uint32_t {
                return epi_h(acc_f(acc[i][jj][v]), xsv[i], wsv[jj][v], et, bsv[jj][v], rv);
            };
            // a residual that is the output itself: each half reads its rows
            // before storing them, and the halves and waves cover disjoint rows
            constexpr int LPR = TN / 8;             // lanes per row
            constexpr int RPI = 64 / LPR;           // rows per store instruction
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int i = hf * FI / 2; i < (hf + 1) * FI / 2; ++i)
#pragma unroll
                    for (int jj = 0; jj < FJ; ++jj)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int64_t o = (int64_t)(m0 + wm * TM + 32 * i + r32) * N + n0 + wn * TN + 32 * jj +
                                              8 * g + 4 * h32;
                            const uint2 rr =
                                et.res ? *reinterpret_cast<const uint2*>(et.res + o) : make_uint2(0u, 0u);
                            uint2 h;
                            h.x = to_h(i, jj, 4 * g, h_lo(rr.x)) | (to_h(i, jj, 4 * g + 1, h_hi(rr.x)) << 16);
                            h.y = to_h(i, jj, 4 * g + 2, h_lo(rr.y)) | (to_h(i, jj, 4 * g + 3, h_hi(rr.y)) << 16);
                            *reinterpret_cast<uint2*>(ot + (32 * (i - hf * FI / 2) + r32) * PITCH + 32 * jj + 8 * g +
                                                      4 * h32) = h;
                        }
                uint16_t* yb = static_cast<uint16_t*>(out) + (int64_t)(m0 + wm * TM + hf * HALF) * N + n0 + wn * TN;
#pragma unroll
                for (int it = 0; it < HALF / RPI; ++it) {
                    const int row = it * RPI + lane / LPR, c = lane % LPR;
                    const uint4 v = *reinterpret_cast<const uint4*>(ot + row * PITCH + 8 * c);
                    *reinterpret_cast<uint4*>(yb + (int64_t)row * N + 8 * c) = v;
                }
            }
            return;
        }
    }
    store_tile32<FI, FJ, kRaw>(acc, xs, ws, et, out, M, N, m0 + wm * TM + r32, n0 + wn * TN + 4 * h32,
                               full && (N & 3) == 0);
}

// Two ring configurations (measured on MI355X, K = 4096):
//   Pipe    -- 256 x 128 tiles, 64-byte k-tiles, 3 stages (72 KiB): two
//              workgroups per CU, so a partial last round of tiles costs little
//   PipeBig -- 256 x 256 tiles, 128-byte k-tiles, 2 stages (128 KiB), 8 waves:
//              a third fewer L2 -> LDS bytes per MFMA, read as whole 128-byte
//              lines, one workgroup per CU
using Pipe = PipeCfg<kQBM, kQBN, 64, 3, true>;
using PipeBig = PipeCfg<256, 256, 128, 2, true, 8>;

// PipeBig where its estimated time is lower.  Measured per-round costs at
// K = 4096 (all scale with K alike): a full round of PipeBig tiles (one per
// CU) 69 us, a partial one ~50-56 us; a full round of Pipe tiles (two per CU)
// 80 us, a partial one of at most one tile per CU ~35 us, a fuller one ~71 us.
// 2048 x 8192: 69 against 80 us; 2048 x 11008 (344 big tiles): 120 against
// 112 us, so Pipe; 4096 x 11008 (688): 192 against 228 us; 1024 x 11008
// (172): 56.5 against 70 us; 3072 x 11008 and 2048 x 16640: equal.
bool use_big_tiles(int64_t m, int64_t n, int64_t k)
{
    if (k % PipeBig::BK || !ql::lds_fits(PipeBig::kLds))
        return false;
    const int64_t cus = ql::cu_count();
    if (cus <= 0)
        return false;
    const int64_t tb = ((m + PipeBig::BM - 1) / PipeBig::BM) * ((n + PipeBig::BN - 1) / PipeBig::BN);
    const int64_t ts = ((m + Pipe::BM - 1) / Pipe::BM) * ((n + Pipe::BN - 1) / Pipe::BN);
    const int64_t big = (tb / cus) * 69 + (tb % cus ? 54 : 0);
    const int64_t rs = ts % (2 * cus);
    const int64_t small = (ts / (2 * cus)) * 80 + (rs == 0 ? 0 : (rs <= cus ? 35 : 75));
    return big < small;
}

template <bool kRaw, bool kF8 = false>
void launch_w8a8_gemm(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws, EpiTerms et,
                      void* out, int64_t m, int64_t n, int64_t k, hipStream_t st)
{
    // grid: whole rounds over the XCDs
    auto grid_for = [&](int bm, int bn) {
        const int64_t tiles = ((n + bn - 1) / bn) * ((m + bm - 1) / bm);
        return (unsigned)((tiles + kXcds - 1) / kXcds * kXcds);
    };
    // the ring kernels address each operand with 32-bit per-lane offsets
    const bool fits32 = m * k < (1LL << 32) && n * k < (1LL << 32);
    if (fits32 && use_big_tiles(m, n, k))
        hipLaunchKernelGGL((w8a8_gemm_pipe_kernel<PipeBig, kRaw, kF8>), dim3(grid_for(PipeBig::BM, PipeBig::BN)),
                           dim3(PipeBig::NW * 64), (size_t)PipeBig::kLds, st, xq, xs, wq, ws, et, out, (int)m, (int)n,
                           (int)k);
    else if (kF8 || (fits32 && k % Pipe::BK == 0 && ql::lds_fits(Pipe::kLds)))   // FP8: checked by the host
        hipLaunchKernelGGL((w8a8_gemm_pipe_kernel<Pipe, kRaw, kF8>), dim3(grid_for(Pipe::BM, Pipe::BN)), dim3(Pipe::NW * 64),
                           (size_t)Pipe::kLds, st, xq, xs, wq, ws, et, out, (int)m, (int)n, (int)k);
    else
        hipLaunchKernelGGL((w8a8_gemm_kernel<kQBM, kQBN, kRaw>), dim3(grid_for(kQBM, kQBN)), dim3(256), 0, st, xq, xs,
                           wq, ws, et, out, (int)m, (int)n, (int)k);
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

namespace {

// Validation and launch shared by the per-token quantisers (one workgroup per
// token; chunks per thread picked from k).
template <int MODE>
int launch_token_quant(const char* who, const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                       float eps, uint16_t* h_out, int8_t* xq, float* x_scale, int64_t m, int64_t k, void* stream)
{
    if (m < 0 || k <= 0 || k % 8)
        QL_FAIL(QL_ERR_SHAPE, "%s: m=%lld k=%lld (k must be a positive multiple of 8)", who, (long long)m,
                (long long)k);
    if (k > 65536 || m > (1LL << 31) - 1)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: k=%lld above 65536", who, (long long)k);
    constexpr bool kNoNorm = MODE == kTokenQuant || MODE == kTokenQuantF8;
    if (!kNoNorm && (!(eps >= 0.0f) || !(eps < 1e30f)))
        QL_FAIL(QL_ERR_VALUE, "%s: eps must be finite and >= 0", who);
    if (m == 0)
        return QL_OK;
    if (!x || !xq || !x_scale || (!kNoNorm && !gamma) || (MODE == kAddNormQuant && (!residual || !h_out)))
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x) || !ql::aligned16(xq) || !ql::aligned16(x_scale) ||
        (!kNoNorm && !ql::aligned16(gamma)) ||
        (MODE == kAddNormQuant && (!ql::aligned16(residual) || !ql::aligned16(h_out))))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    const int64_t cpt = (k / 8 + kNormThreads - 1) / kNormThreads;   // 16-byte chunks per thread
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)m), block(kNormThreads);
    const int ki = (int)k;
    // QRMSNorm of short tokens (k from 2049 to 4096) on 128 threads with four
    // chunks each: the per-token reductions, divisions and square root are
    // then paid by half as many waves (2048 x 4096: 8.4 -> 8.0 us; the
    // quantisers without the norm and the residual-add form are faster on 256)
    if constexpr (MODE == kNormQuant || MODE == kNormQuantF8) {
        if (k > 2048 && k <= 4096) {
            hipLaunchKernelGGL((quant_rmsnorm_kernel<4, MODE, 128>), grid, dim3(128), 0, st, x, residual, gamma, eps,
                               h_out, xq, x_scale, ki);
            return launch_status(who);
        }
    }
    if (cpt <= 1)
        hipLaunchKernelGGL((quant_rmsnorm_kernel<1, MODE>), grid, block, 0, st, x, residual, gamma, eps, h_out, xq,
                           x_scale, ki);
    else if (cpt <= 2)
        hipLaunchKernelGGL((quant_rmsnorm_kernel<2, MODE>), grid, block, 0, st, x, residual, gamma, eps, h_out, xq,
                           x_scale, ki);
    else if (cpt <= 4)
        hipLaunchKernelGGL((quant_rmsnorm_kernel<4, MODE>), grid, block, 0, st, x, residual, gamma, eps, h_out, xq,
                           x_scale, ki);
    else if (cpt <= 8)
        hipLaunchKernelGGL((quant_rmsnorm_kernel<8, MODE>), grid, block, 0, st, x, residual, gamma, eps, h_out, xq,
                           x_scale, ki);
    else
        hipLaunchKernelGGL((quant_rmsnorm_kernel<0, MODE>), grid, block, 0, st, x, residual, gamma, eps, h_out, xq,
                           x_scale, ki);
    return launch_status(who);
}

}  // namespace

extern "C" int ql_w8a8_quant_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int8_t* xq,
                                     float* x_scale, int64_t m, int64_t k, void* stream)
{
    ql::clear_error();
    return launch_token_quant<kNormQuant>("ql_w8a8_quant_rmsnorm", x, nullptr, gamma, eps, nullptr, xq, x_scale, m, k,
                                          stream);
}

extern "C" int ql_w8a8_add_quant_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                                         float eps, uint16_t* h_out, int8_t* xq, float* x_scale, int64_t m,
                                         int64_t k, void* stream)
{
    ql::clear_error();
    return launch_token_quant<kAddNormQuant>("ql_w8a8_add_quant_rmsnorm", x, residual, gamma, eps, h_out, xq,
                                             x_scale, m, k, stream);
}

extern "C" int ql_w8a8_quant_per_token(const uint16_t* x, int8_t* xq, float* x_scale, int64_t m, int64_t k,
                                       void* stream)
{
    ql::clear_error();
    return launch_token_quant<kTokenQuant>("ql_w8a8_quant_per_token", x, nullptr, nullptr, 0.0f, nullptr, xq,
                                           x_scale, m, k, stream);
}

extern "C" int ql_fp8_quant_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, uint8_t* xq,
                                    float* x_scale, int64_t m, int64_t k, void* stream)
{
    ql::clear_error();
    return launch_token_quant<kNormQuantF8>("ql_fp8_quant_rmsnorm", x, nullptr, gamma, eps, nullptr,
                                            reinterpret_cast<int8_t*>(xq), x_scale, m, k, stream);
}

extern "C" int ql_fp8_quant_per_token(const uint16_t* x, uint8_t* xq, float* x_scale, int64_t m, int64_t k,
                                      void* stream)
{
    ql::clear_error();
    return launch_token_quant<kTokenQuantF8>("ql_fp8_quant_per_token", x, nullptr, nullptr, 0.0f, nullptr,
                                             reinterpret_cast<int8_t*>(xq), x_scale, m, k, stream);
}

namespace {

int w8a8_gemm_fp16(const char* who, const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                   const uint16_t* bias, const uint16_t* residual, uint16_t* y, int64_t m, int64_t n, int64_t k,
                   void* stream)
{
    if (int rc = check_gemm(xq, wq, y, m, n, k, who))
        return rc;
    if (m == 0 || n == 0)
        return QL_OK;
    if (!x_scale || !w_scale)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x_scale) || !ql::aligned16(w_scale) || (bias && !ql::aligned16(bias)) ||
        (residual && !ql::aligned16(residual)))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    launch_w8a8_gemm<false>(xq, x_scale, wq, w_scale, EpiTerms{bias, residual}, (void*)y, m, n, k,
                            static_cast<hipStream_t>(stream));
    return launch_status(who);
}

}  // namespace

extern "C" int ql_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                            uint16_t* y, int64_t m, int64_t n, int64_t k, void* stream)
{
    ql::clear_error();
    return w8a8_gemm_fp16("ql_w8a8_gemm", xq, x_scale, wq, w_scale, nullptr, nullptr, y, m, n, k, stream);
}

extern "C" int ql_w8a8_gemm_ex(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                               const uint16_t* bias, const uint16_t* residual, uint16_t* y, int64_t m, int64_t n,
                               int64_t k, void* stream)
{
    ql::clear_error();
    return w8a8_gemm_fp16("ql_w8a8_gemm_ex", xq, x_scale, wq, w_scale, bias, residual, y, m, n, k, stream);
}

extern "C" int ql_fp8_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                           const uint16_t* bias, const uint16_t* residual, uint16_t* y, int64_t m, int64_t n,
                           int64_t k, void* stream)
{
    ql::clear_error();
    const char* who = "ql_fp8_gemm";
    if (int rc = check_gemm(xq, wq, y, m, n, k, who))
        return rc;
    if (k % Pipe::BK)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: k=%lld (the FP8 GEMM needs a multiple of 64)", who, (long long)k);
    if (m * k >= (1LL << 32) || n * k >= (1LL << 32))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: operands of 4 GiB or more (m=%lld n=%lld k=%lld)", who, (long long)m,
                (long long)n, (long long)k);
    if (m == 0 || n == 0)
        return QL_OK;
    if (!x_scale || !w_scale)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x_scale) || !ql::aligned16(w_scale) || (bias && !ql::aligned16(bias)) ||
        (residual && !ql::aligned16(residual)))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    if (!ql::lds_fits(Pipe::kLds))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: the device lacks the LDS the FP8 GEMM needs", who);
    launch_w8a8_gemm<false, true>(reinterpret_cast<const int8_t*>(xq), x_scale, reinterpret_cast<const int8_t*>(wq),
                                  w_scale, EpiTerms{bias, residual}, (void*)y, m, n, k,
                                  static_cast<hipStream_t>(stream));
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
    launch_w8a8_gemm<true>(xq, nullptr, wq, nullptr, EpiTerms{nullptr, nullptr}, (void*)acc, m, n, k,
                           static_cast<hipStream_t>(stream));
    return launch_status(who);
}
