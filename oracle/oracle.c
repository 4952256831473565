/*
 * oracle.c -- plain, slow CPU reference of the quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product (libqlinear
 * and its Python binding) never calls it, and the two share no source: this
 * file includes no project header and defines its own half-precision codec.
 *
 * What it computes, step by step, and where each step comes from:
 *
 *   W4A16 (AWQ-style weight-only int4), LMDeploy walkthrough, section 2
 *   ("quantization is not trading precision for speed"): per-group scales
 *   along the input dimension, an asymmetric zero point from each group's
 *   min/max, 4-bit codes; AUQ dual-process page, sections 3.3 and 5.4: the
 *   qweight / scales / zeros tensors and the "int4 times scale, zero point"
 *   dequantisation.
 *     1. lo = min(0, min w), hi = max(0, max w) over a group of G weights.
 *     2. s = fp16 rounded toward +inf of max((hi - lo) / 15, 2^-14).
 *     3. z = clamp(rint(-lo / s), 0, 15).
 *     4. q = clamp(rint(w / s) + z, 0, 15).
 *     5. 8 codes per 32-bit word, code i in bits [4i, 4i+4), along K.
 *     6. unpack = the inverse of 5.
 *     7. wd = (q - z) * s (exact in fp32); wd16 = its fp16 rounding.
 *     8. y[m,n] = sum_k x[m,k] * wd16[n,k], fp64 accumulator, k ascending.
 *   The symmetric per-tensor example of the same section (scale = max|w| /
 *   7.5, codes clamped to [-7, 7]) is implemented as or_sym_int4.
 *
 *   W8A8 (SmoothQuant), LMDeploy W8A8 guide, "step 2: weight smoothing" and
 *   "inference kernels: QRMSNorm and QLinear":
 *     1. a_j = max_m |X[m,j]|, b_j = max_n |W[n,j]|,
 *        s_j = a_j^0.5 / b_j^0.5 (alpha = 0.5); s_j = 1 where a_j, b_j or
 *        gamma_j is zero.
 *     2. gamma'_j = fp16(gamma_j / s_j); W'[n,j] = W[n,j] * s_j.
 *     3. per output channel: w_scale = max_j |W'| / 127,
 *        wq = clamp(rint(W' / w_scale), -127, 127).
 *     4. per token: RMSNorm y = x * (1/sqrt(mean(x^2) + eps)) * gamma' in
 *        fp32, x_scale = max|y| / 127, xq = clamp(rint(y / x_scale), -127, 127).
 *        mean(x^2) is the exact mean rounded once to fp32.
 *     5. acc = sum_j xq * wq in exact integer arithmetic.
 *     6. y = acc * x_scale * w_scale (fp64).
 *   The same guide's kernel list adds the steps on either side of the path:
 *     7. residual fusion of the norm: h = fp16(x + residual), the new
 *        residual stream, then step 4 on h.
 *     8. per-token quantisation of a plain activation (a QLinear whose input
 *        did not come from QRMSNorm): x_scale = max|x| / 127,
 *        xq = clamp(rint(x / x_scale), -127, 127).
 *     9. the GEMM epilogue with an optional bias [n] and residual [m, n]:
 *        y = acc * x_scale * w_scale + bias + residual (fp64).
 *   The guide's second 8-bit type, float8_e4m3fn (--quant-dtype fp8), takes
 *   the same steps with Q_MAX = the format's largest finite value, 448, and
 *   a cast to the format in place of rint + clamp:
 *    10. per token x_scale = max|y| / 448, xq = e4m3(y / x_scale); per output
 *        channel w_scale = max|W'| / 448, wq = e4m3(W' / w_scale).
 *    11. acc = sum_j e4m3 value of xq * e4m3 value of wq (exact products,
 *        fp64 sum), y = acc * x_scale * w_scale (fp64).
 *
 *   KV cache INT8 (FastLLM architecture page, section 5.2: KV cache group
 *   quantisation between FP16 and INT8, groups of 128):
 *    12. per group of G consecutive values (a head's vector at G = 128):
 *        scale = max|x| / 127, q = clamp(rint(x / scale), -127, 127);
 *        dequantisation x' = fp16(fp32(q * scale)).
 *
 *   e4m3 (OCP FP8 E4M3, "fn": no infinities): sign, 4 exponent bits with bias
 *   7, 3 fraction bits; exponent field 0 is subnormal (fraction * 2^-9); the
 *   all-ones pattern S.1111.111 is NaN, so the largest finite value is
 *   1.75 * 2^8 = 448.  The cast rounds to nearest, ties to even; magnitudes
 *   above 464 (halfway to the next step) become NaN.
 *
 *   AWQ scale search (LMDeploy walkthrough, section 2: AWQ samples typical
 *   inputs and picks the scales that minimise the error of the product with
 *   those activations, not of the weights; LMDeploy W8A8 guide, source
 *   analysis of the smoothing: coefficient act_scales^alpha /
 *   w_scales^(1 - alpha), with per-layer ratios found in calibration
 *   replacing the fixed alpha when the scale search is on):
 *    13. a_j = max_t |x[t,j]| over the calibration tokens, b_j = max_r |w[r,j]|.
 *    14. for alpha = i / grid, i = 0 .. grid-1:
 *        s_j = exp(alpha ln a_j - (1 - alpha) ln b_j) in fp64, rounded to
 *        fp32 (s_j = 1 where a_j or b_j is zero); W' = W diag(s) (fp32),
 *        quantised and dequantised to fp16 by steps 1-4 and 7;
 *        x' = fp16(fp32(x) / s_j);  y = fp16 of the fp64 sum x' wd16^T
 *        (the precision the device GEMM delivers its output in);
 *        err_i = sum over (t, r) of (y - yref)^2, yref = x W^T in fp64.
 *    15. the chosen ratio is the first i with the smallest err_i.
 *
 * Rounding: rintf under the default environment (nearest, ties to even).
 * Built with -ffp-contract=off so every fp32 operation rounds on its own.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD -1

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"), from the format's definition                     */
/* ------------------------------------------------------------------------ */

float or_e4m3_to_f32(uint8_t b)
{
    const int sgn = b >> 7, e = (b >> 3) & 15, f = b & 7;
    float v;
    if (e == 15 && f == 7)
        return sgn ? -NAN : NAN;
    if (e == 0)
        v = ldexpf((float)f, -9);
    else
        v = ldexpf(1.0f + (float)f / 8.0f, e - 7);
    return sgn ? -v : v;
}

/* Values of the non-negative finite codes 0..126 (increasing with the code). */
static float e4m3_val[127];
static int e4m3_ready;
static void e4m3_init(void)
{
    if (e4m3_ready)
        return;
    for (int c = 0; c < 127; ++c)
        e4m3_val[c] = or_e4m3_to_f32((uint8_t)c);
    e4m3_ready = 1;
}

/* float32 -> e4m3, nearest with ties to even: find the code just below |x|
 * (binary search over the increasing code values), then step up if |x| lies
 * past the midpoint to the next code, or on it with an odd code below (the
 * midpoint is exact in fp32: adjacent codes differ by a power of two).
 * e4m3_init() must have run. */
static uint8_t f32_to_e4m3(float x)
{
    const uint8_t sgn = signbit(x) ? 0x80 : 0;
    const float a = fabsf(x);
    if (isnan(x) || a > 464.0f)
        return (uint8_t)(sgn | 0x7F);
    if (a >= 448.0f)
        return (uint8_t)(sgn | 0x7E);
    int lo = 0, hi = 126;                         /* e4m3_val[lo] <= a < e4m3_val[hi] */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (e4m3_val[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    const float half = e4m3_val[lo] + (e4m3_val[lo + 1] - e4m3_val[lo]) / 2.0f;
    int c = lo;
    if (a > half || (a == half && (lo & 1)))
        c = lo + 1;
    return (uint8_t)(sgn | c);
}

uint8_t or_f32_to_e4m3(float x)
{
    e4m3_init();
    return f32_to_e4m3(x);
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16, from the format's definition                           */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> value.  sign | 5-bit biased exponent | 10-bit fraction. */
float or_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(f | 0x400), e - 25);    /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* value -> binary16 bits, rounding to nearest, ties to even. */
uint16_t or_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    float a = fabsf(x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0f)              /* halfway above 65504 and beyond: overflow */
        return sign | 0x7c00;
    if (a < ldexpf(1.0f, -14)) {    /* subnormal range: quantum 2^-24 */
        float m = rintf(ldexpf(a, 24));
        return sign | (uint16_t)m;  /* m == 1024 encodes the smallest normal */
    }
    int e2;
    frexpf(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
    int ex = e2 - 1;                /* a in [2^ex, 2^(ex+1)) */
    float m = rintf(ldexpf(a, 10 - ex));   /* significand in [1024, 2048] */
    if (m == 2048.0f) {
        m = 1024.0f;
        ex += 1;
    }
    if (ex + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)m - 1024));
}

/* the same rounding from a binary64 value (scaling by powers of two is exact,
 * so the one rint is the only rounding) */
uint16_t or_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        double m = rint(ldexp(a, 24));
        return sign | (uint16_t)m;
    }
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    double m = rint(ldexp(a, 10 - ex));
    if (m == 2048.0) {
        m = 1024.0;
        ex += 1;
    }
    if (ex + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)m - 1024));
}

/* smallest binary16 value >= x, for finite x >= 2^-14 */
uint16_t or_f32_to_f16_up(float x)
{
    uint16_t h = or_f32_to_f16(x);
    if (or_f16_to_f32(h) < x)
        h = (uint16_t)(h + 1);      /* next representable value up (x > 0) */
    return h;
}

/* element-wise forms of the three conversions above, for arrays */
void or_f16_to_f32_n(const uint16_t* h, int64_t count, float* out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = or_f16_to_f32(h[i]);
}

void or_f32_to_f16_n(const float* x, int64_t count, int round_up, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = round_up ? or_f32_to_f16_up(x[i]) : or_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* W4A16: group-wise asymmetric uint4                                        */
/* ------------------------------------------------------------------------ */

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/*
 * Steps 1-4.  w: float32 [n, k] row-major.  Outputs q uint8 [n, k] (codes),
 * z uint8 [n, k/G] (zero points), s uint16 [n, k/G] (fp16 scale bits).
 */
int or_awq_quantize(const float* w, int64_t n, int64_t k, int G,
                    uint8_t* q, uint8_t* z, uint16_t* s)
{
    if (G <= 0 || k % G)
        return OR_BAD;
    const int64_t ng = k / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const float* wg = w + r * k + g * G;
            float lo = 0.0f, hi = 0.0f;
            for (int i = 0; i < G; ++i) {
                if (wg[i] < lo) lo = wg[i];
                if (wg[i] > hi) hi = wg[i];
            }
            float step = (hi - lo) / 15.0f;
            float floor_s = ldexpf(1.0f, -14);
            if (step < floor_s)
                step = floor_s;
            uint16_t sb = or_f32_to_f16_up(step);
            float sv = or_f16_to_f32(sb);
            int zp = clampi((int)rintf(-lo / sv), 0, 15);
            s[r * ng + g] = sb;
            z[r * ng + g] = (uint8_t)zp;
            for (int i = 0; i < G; ++i)
                q[r * k + g * G + i] = (uint8_t)clampi((int)rintf(wg[i] / sv) + zp, 0, 15);
        }
    }
    return OR_OK;
}

/* Step 5.  qweight uint32 [n, k/8]; qzeros uint32 [n, ceil((k/G)/8)], pad 0. */
int or_awq_pack(const uint8_t* q, const uint8_t* z, int64_t n, int64_t k, int G,
                uint32_t* qweight, uint32_t* qzeros)
{
    if (k % 8 || G <= 0 || k % G)
        return OR_BAD;
    const int64_t ng = k / G, zw = (ng + 7) / 8;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < k / 8; ++j) {
            uint32_t word = 0;
            for (int i = 0; i < 8; ++i)
                word |= (uint32_t)(q[r * k + 8 * j + i] & 0xF) << (4 * i);
            qweight[r * (k / 8) + j] = word;
        }
        for (int64_t v = 0; v < zw; ++v) {
            uint32_t word = 0;
            for (int i = 0; i < 8; ++i) {
                int64_t g = 8 * v + i;
                if (g < ng)
                    word |= (uint32_t)(z[r * ng + g] & 0xF) << (4 * i);
            }
            qzeros[r * zw + v] = word;
        }
    }
    return OR_OK;
}

/* Step 6. */
int or_awq_unpack(const uint32_t* qweight, const uint32_t* qzeros, int64_t n, int64_t k, int G,
                  uint8_t* q, uint8_t* z)
{
    if (k % 8 || G <= 0 || k % G)
        return OR_BAD;
    const int64_t ng = k / G, zw = (ng + 7) / 8;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c)
            q[r * k + c] = (uint8_t)((qweight[r * (k / 8) + c / 8] >> (4 * (c % 8))) & 0xF);
        for (int64_t g = 0; g < ng; ++g)
            z[r * ng + g] = (uint8_t)((qzeros[r * zw + g / 8] >> (4 * (g % 8))) & 0xF);
    }
    return OR_OK;
}

/* Step 7.  wd float32 [n, k] (nullable), wd16 fp16 bits [n, k] (nullable). */
int or_awq_dequant(const uint8_t* q, const uint8_t* z, const uint16_t* s,
                   int64_t n, int64_t k, int G, float* wd, uint16_t* wd16)
{
    if (G <= 0 || k % G)
        return OR_BAD;
    const int64_t ng = k / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            int64_t g = c / G;
            float v = (float)((int)q[r * k + c] - (int)z[r * ng + g]) * or_f16_to_f32(s[r * ng + g]);
            if (wd)
                wd[r * k + c] = v;
            if (wd16)
                wd16[r * k + c] = or_f32_to_f16(v);
        }
    }
    return OR_OK;
}

/*
 * Step 8.  x fp16 [m, k]; wd16 fp16 [n, k].  y float64 [m, nrows] for the
 * output channels listed in rows (all n channels when rows is NULL).
 */
int or_w4a16_matmul(const uint16_t* x, int64_t m, const uint16_t* wd16, int64_t n, int64_t k,
                    const int64_t* rows, int64_t nrows, double* y)
{
    if (!rows)
        nrows = n;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        if (r < 0 || r >= n)
            continue;
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c)
                acc += (double)or_f16_to_f32(x[i * k + c]) * (double)or_f16_to_f32(wd16[r * k + c]);
            y[i * nrows + j] = acc;
        }
    }
    return OR_OK;
}

/*
 * Steps 6-8 from the packed tensors for a subset of output channels: unpack,
 * dequantise and contract one channel at a time.
 */
int or_w4a16_forward(const uint16_t* x, int64_t m, const uint32_t* qweight, const uint16_t* scales,
                     const uint32_t* qzeros, int64_t n, int64_t k, int G,
                     const int64_t* rows, int64_t nrows, double* y)
{
    if (k % 8 || G <= 0 || k % G)
        return OR_BAD;
    if (!rows)
        nrows = n;
    const int64_t ng = k / G, zw = (ng + 7) / 8;
    int bad = 0;
#pragma omp parallel
    {
        uint8_t* q = (uint8_t*)malloc((size_t)k);
        uint8_t* z = (uint8_t*)malloc((size_t)ng);
        uint16_t* w16 = (uint16_t*)malloc((size_t)k * 2);
        if (!q || !z || !w16) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t j = 0; j < nrows; ++j) {
                int64_t r = rows ? rows[j] : j;
                if (r < 0 || r >= n)
                    continue;
                or_awq_unpack(qweight + r * (k / 8), qzeros + r * zw, 1, k, G, q, z);
                or_awq_dequant(q, z, scales + r * ng, 1, k, G, NULL, w16);
                for (int64_t i = 0; i < m; ++i) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < k; ++c)
                        acc += (double)or_f16_to_f32(x[i * k + c]) * (double)or_f16_to_f32(w16[c]);
                    y[i * nrows + j] = acc;
                }
            }
        }
        free(q);
        free(z);
        free(w16);
    }
    return bad ? OR_BAD : OR_OK;
}

/* Symmetric per-tensor int4 of the worked example: scale = max|w| / 7.5. */
int or_sym_int4(const float* w, int64_t count, float* scale_out, int8_t* q)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < count; ++i)
        if (fabsf(w[i]) > amax)
            amax = fabsf(w[i]);
    float scale = amax / 7.5f;
    *scale_out = scale;
    if (q)
        for (int64_t i = 0; i < count; ++i)
            q[i] = (int8_t)(scale > 0.0f ? clampi((int)rintf(w[i] / scale), -7, 7) : 0);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* W8A8: SmoothQuant smoothing, int8 weights, QRMSNorm, integer GEMM          */
/* ------------------------------------------------------------------------ */

/*
 * Steps 1-2.  x fp16 [rows, k] (calibration activations), gamma fp16 [k],
 * w float32 [n, k].  Outputs s float32 [k], gamma_s fp16 [k], w_s float32 [n, k].
 */
int or_smooth(const uint16_t* x, int64_t rows, const uint16_t* gamma, const float* w,
              int64_t n, int64_t k, float* s, uint16_t* gamma_s, float* w_s)
{
    for (int64_t j = 0; j < k; ++j) {
        float a = 0.0f, b = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            float v = fabsf(or_f16_to_f32(x[r * k + j]));
            if (v > a) a = v;
        }
        for (int64_t r = 0; r < n; ++r) {
            float v = fabsf(w[r * k + j]);
            if (v > b) b = v;
        }
        float g = or_f16_to_f32(gamma[j]);
        float sj = (a == 0.0f || b == 0.0f || g == 0.0f) ? 1.0f : sqrtf(a) / sqrtf(b);
        s[j] = sj;
        gamma_s[j] = or_f32_to_f16(g / sj);
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j)
            w_s[r * k + j] = w[r * k + j] * s[j];
    return OR_OK;
}

/* Step 3.  wq int8 [n, k], w_scale float32 [n]. */
int or_w8_quant_weight(const float* w, int64_t n, int64_t k, int8_t* wq, float* w_scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j)
            if (fabsf(w[r * k + j]) > amax)
                amax = fabsf(w[r * k + j]);
        float sc = amax / 127.0f;
        w_scale[r] = sc;
        for (int64_t j = 0; j < k; ++j)
            wq[r * k + j] = (int8_t)(sc > 0.0f ? clampi((int)rintf(w[r * k + j] / sc), -127, 127) : 0);
    }
    return OR_OK;
}

/*
 * Exact sum of squares of fp16 values as an unsigned 128-bit integer in units
 * of 2^-48.  An fp16 value is an integer significand times 2^(e-25); its
 * square is significand^2 * 2^(2e-50) = (significand^2 << (2e-2)) * 2^-48.
 */
static unsigned __int128 sumsq_exact(const uint16_t* x, int64_t k)
{
    unsigned __int128 acc = 0;
    for (int64_t j = 0; j < k; ++j) {
        uint16_t h = x[j];
        int e = (h >> 10) & 0x1f;
        uint64_t sig = h & 0x3ff;
        if (e == 0)
            e = 1;
        else
            sig |= 0x400;
        acc += (unsigned __int128)(sig * sig) << (2 * e - 2);
    }
    return acc;
}

static int bitlen128(unsigned __int128 v)
{
    int b = 0;
    while (v) {
        v >>= 1;
        ++b;
    }
    return b;
}

/*
 * num / den * 2^e2 rounded to the nearest fp32 (ties to even).  The result
 * must lie in the normal fp32 range (true for the mean of squares below).
 */
float or_ratio_to_f32(unsigned __int128 num, uint64_t den, int e2)
{
    if (num == 0)
        return 0.0f;
    /* choose t so that q = floor(num * 2^t / den) has exactly 25 bits */
    int t = 25 - (bitlen128(num) - bitlen128(den));
    unsigned __int128 qv, rv;
    for (;;) {
        unsigned __int128 a = t >= 0 ? num << t : num;
        unsigned __int128 b = t >= 0 ? (unsigned __int128)den : (unsigned __int128)den << (-t);
        qv = a / b;
        rv = a % b;
        int bl = bitlen128(qv);
        if (bl == 25)
            break;
        t += (bl < 25) ? 1 : -1;
    }
    uint32_t mant = (uint32_t)(qv >> 1);        /* 24 significant bits */
    int rbit = (int)(qv & 1);
    int sticky = rv != 0;
    if (rbit && (sticky || (mant & 1)))
        ++mant;                                 /* 2^24 after a carry is still exact */
    return ldexpf((float)mant, e2 - t + 1);
}

/*
 * Step 4 for m tokens.  x fp16 [m, k], gamma fp16 [k] (already smoothed).
 * xq int8 [m, k], x_scale float32 [m], ms_out float32 [m] (nullable: the
 * rounded mean of squares, exposed for the pins).
 */
int or_quant_rmsnorm(const uint16_t* x, int64_t m, int64_t k, const uint16_t* gamma, float eps,
                     int8_t* xq, float* x_scale, float* ms_out)
{
    if (k <= 0)
        return OR_BAD;
    int bad = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc((size_t)k * sizeof(float));
        if (!y) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; ++i) {
                const uint16_t* xr = x + i * k;
                float ms = or_ratio_to_f32(sumsq_exact(xr, k), (uint64_t)k, -48);
                float r = 1.0f / sqrtf(ms + eps);
                float amax = 0.0f;
                for (int64_t j = 0; j < k; ++j) {
                    float t = or_f16_to_f32(xr[j]) * r;
                    y[j] = t * or_f16_to_f32(gamma[j]);
                    if (fabsf(y[j]) > amax)
                        amax = fabsf(y[j]);
                }
                float sc = amax / 127.0f;
                x_scale[i] = sc;
                if (ms_out)
                    ms_out[i] = ms;
                for (int64_t j = 0; j < k; ++j)
                    xq[i * k + j] = (int8_t)(sc > 0.0f ? clampi((int)rintf(y[j] / sc), -127, 127) : 0);
            }
        }
        free(y);
    }
    return bad ? OR_BAD : OR_OK;
}

/*
 * Step 7 for m tokens: h = fp16(x + residual) element by element, then step 4
 * on h.  The fp32 sum of two binary16 values rounded to binary16 is the
 * correctly rounded sum (24 >= 2 * 11 + 2 bits, so the double rounding is
 * innocuous).  h fp16 [m, k] (written; may not alias x or residual here).
 */
int or_add_quant_rmsnorm(const uint16_t* x, const uint16_t* residual, int64_t m, int64_t k,
                         const uint16_t* gamma, float eps, uint16_t* h, int8_t* xq, float* x_scale,
                         float* ms_out)
{
    if (k <= 0)
        return OR_BAD;
    for (int64_t i = 0; i < m * k; ++i)
        h[i] = or_f32_to_f16(or_f16_to_f32(x[i]) + or_f16_to_f32(residual[i]));
    return or_quant_rmsnorm(h, m, k, gamma, eps, xq, x_scale, ms_out);
}

/*
 * Step 8 for m tokens: x fp16 [m, k] -> xq int8 [m, k], x_scale float32 [m].
 * The scale and the quotient are fp32 divisions; a zero row gets scale 0 and
 * codes 0.
 */
int or_quant_per_token(const uint16_t* x, int64_t m, int64_t k, int8_t* xq, float* x_scale)
{
    if (k <= 0)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const uint16_t* xr = x + i * k;
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j)
            if (fabsf(or_f16_to_f32(xr[j])) > amax)
                amax = fabsf(or_f16_to_f32(xr[j]));
        float sc = amax / 127.0f;
        x_scale[i] = sc;
        for (int64_t j = 0; j < k; ++j)
            xq[i * k + j] = (int8_t)(sc > 0.0f ? clampi((int)rintf(or_f16_to_f32(xr[j]) / sc), -127, 127) : 0);
    }
    return OR_OK;
}

/*
 * Step 5 on a sub-grid: acc int64 [nr, nc] for rows[] x cols[] (all when NULL).
 */
int or_int8_gemm(const int8_t* xq, int64_t m, const int8_t* wq, int64_t n, int64_t k,
                 const int64_t* rows, int64_t nr, const int64_t* cols, int64_t nc, int64_t* acc)
{
    if (!rows)
        nr = m;
    if (!cols)
        nc = n;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t a = 0; a < nr; ++a) {
        int64_t i = rows ? rows[a] : a;
        for (int64_t b = 0; b < nc; ++b) {
            int64_t j = cols ? cols[b] : b;
            int64_t s = 0;
            if (i >= 0 && i < m && j >= 0 && j < n)
                for (int64_t c = 0; c < k; ++c)
                    s += (int64_t)xq[i * k + c] * (int64_t)wq[j * k + c];
            acc[a * nc + b] = s;
        }
    }
    return OR_OK;
}

/* Steps 5-6 on a sub-grid: y float64 [nr, nc]. */
int or_w8a8_forward(const int8_t* xq, const float* x_scale, int64_t m, const int8_t* wq,
                    const float* w_scale, int64_t n, int64_t k,
                    const int64_t* rows, int64_t nr, const int64_t* cols, int64_t nc, double* y)
{
    if (!rows)
        nr = m;
    if (!cols)
        nc = n;
    int64_t* acc = (int64_t*)malloc((size_t)(nr * nc) * sizeof(int64_t));
    if (!acc)
        return OR_BAD;
    or_int8_gemm(xq, m, wq, n, k, rows, nr, cols, nc, acc);
    for (int64_t a = 0; a < nr; ++a) {
        int64_t i = rows ? rows[a] : a;
        for (int64_t b = 0; b < nc; ++b) {
            int64_t j = cols ? cols[b] : b;
            y[a * nc + b] = (double)acc[a * nc + b] * (double)x_scale[i] * (double)w_scale[j];
        }
    }
    free(acc);
    return OR_OK;
}

/*
 * Step 9 on a sub-grid: steps 5-6 plus bias fp16 [n] and residual fp16
 * [m, n] (either may be NULL), y float64 [nr, nc].
 */
int or_w8a8_forward_ex(const int8_t* xq, const float* x_scale, int64_t m, const int8_t* wq,
                       const float* w_scale, int64_t n, int64_t k, const uint16_t* bias,
                       const uint16_t* residual, const int64_t* rows, int64_t nr, const int64_t* cols,
                       int64_t nc, double* y)
{
    if (!rows)
        nr = m;
    if (!cols)
        nc = n;
    int rc = or_w8a8_forward(xq, x_scale, m, wq, w_scale, n, k, rows, nr, cols, nc, y);
    if (rc != OR_OK)
        return rc;
    for (int64_t a = 0; a < nr; ++a) {
        int64_t i = rows ? rows[a] : a;
        for (int64_t b = 0; b < nc; ++b) {
            int64_t j = cols ? cols[b] : b;
            if (bias)
                y[a * nc + b] += (double)or_f16_to_f32(bias[j]);
            if (residual)
                y[a * nc + b] += (double)or_f16_to_f32(residual[i * n + j]);
        }
    }
    return OR_OK;
}

/*
 * Step 10, activations: RMSNorm as step 4 (or y = x without the norm when
 * gamma is NULL), x_scale = max|y| / 448, xq = e4m3(y / x_scale) (bytes).
 */
int or_quant_fp8(const uint16_t* x, int64_t m, int64_t k, const uint16_t* gamma, float eps, uint8_t* xq,
                 float* x_scale)
{
    if (k <= 0)
        return OR_BAD;
    e4m3_init();
    int bad = 0;
#pragma omp parallel
    {
        float* y = (float*)malloc((size_t)k * sizeof(float));
        if (!y) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; ++i) {
                const uint16_t* xr = x + i * k;
                float r = 1.0f;
                if (gamma) {
                    float ms = or_ratio_to_f32(sumsq_exact(xr, k), (uint64_t)k, -48);
                    r = 1.0f / sqrtf(ms + eps);
                }
                float amax = 0.0f;
                for (int64_t j = 0; j < k; ++j) {
                    y[j] = gamma ? (or_f16_to_f32(xr[j]) * r) * or_f16_to_f32(gamma[j]) : or_f16_to_f32(xr[j]);
                    if (fabsf(y[j]) > amax)
                        amax = fabsf(y[j]);
                }
                float sc = amax / 448.0f;
                x_scale[i] = sc;
                for (int64_t j = 0; j < k; ++j)
                    xq[i * k + j] = sc > 0.0f ? f32_to_e4m3(y[j] / sc) : 0;
            }
        }
        free(y);
    }
    return bad ? OR_BAD : OR_OK;
}

/* Step 10, weights: per output channel w_scale = max_j |W'| / 448,
 * wq = e4m3(W' / w_scale); an all-zero row gets codes 0 and scale 0. */
int or_fp8_quant_weight(const float* w, int64_t n, int64_t k, uint8_t* wq, float* w_scale)
{
    e4m3_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j)
            if (fabsf(w[i * k + j]) > amax)
                amax = fabsf(w[i * k + j]);
        float sc = amax / 448.0f;
        w_scale[i] = sc;
        for (int64_t j = 0; j < k; ++j)
            wq[i * k + j] = sc > 0.0f ? f32_to_e4m3(w[i * k + j] / sc) : 0;
    }
    return OR_OK;
}

/* Step 11 on a sub-grid: y float64 [nr, nc] (acc alone when the scales are NULL). */
int or_fp8_forward(const uint8_t* xq, const float* x_scale, int64_t m, const uint8_t* wq, const float* w_scale,
                   int64_t n, int64_t k, const int64_t* rows, int64_t nr, const int64_t* cols, int64_t nc, double* y)
{
    if (!rows)
        nr = m;
    if (!cols)
        nc = n;
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = (double)or_e4m3_to_f32((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t a = 0; a < nr; ++a) {
        int64_t i = rows ? rows[a] : a;
        for (int64_t b = 0; b < nc; ++b) {
            int64_t j = cols ? cols[b] : b;
            double s = 0.0;
            for (int64_t c = 0; c < k; ++c)
                s += lut[xq[i * k + c]] * lut[wq[j * k + c]];
            y[a * nc + b] = (x_scale && w_scale) ? s * (double)x_scale[i] * (double)w_scale[j] : s;
        }
    }
    return OR_OK;
}

/* Step 12: x fp16 [groups * G] -> q int8 [groups * G], scale float32 [groups]
 * (fp32 divisions; a zero group gets scale 0 and codes 0). */
int or_kv_quant_int8(const uint16_t* x, int64_t groups, int G, int8_t* q, float* scale)
{
    if (G <= 0)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < groups; ++g) {
        const uint16_t* xg = x + g * G;
        float amax = 0.0f;
        for (int j = 0; j < G; ++j)
            if (fabsf(or_f16_to_f32(xg[j])) > amax)
                amax = fabsf(or_f16_to_f32(xg[j]));
        const float sc = amax / 127.0f;
        scale[g] = sc;
        for (int j = 0; j < G; ++j)
            q[g * G + j] = (int8_t)(sc > 0.0f ? clampi((int)rintf(or_f16_to_f32(xg[j]) / sc), -127, 127) : 0);
    }
    return OR_OK;
}

/* Step 12, dequantisation: out fp16 = fp16(fp32(q * scale)), the fp32
 * product cast to binary16 (two roundings: the product of an 8-bit code and a
 * 24-bit scale need not be exact in fp32). */
int or_kv_dequant_int8(const int8_t* q, const float* scale, int64_t groups, int G, uint16_t* out)
{
    if (G <= 0)
        return OR_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < groups; ++g)
        for (int j = 0; j < G; ++j)
            out[g * G + j] = or_f32_to_f16((float)q[g * G + j] * scale[g]);
    return OR_OK;
}

/* Threads the OpenMP loops of this file use. */
int or_num_threads(void) { return omp_get_max_threads(); }

/* Exposed for the pins: exact sum of squares as (hi, lo) 64-bit halves. */
void or_sumsq_exact(const uint16_t* x, int64_t k, uint64_t* hi, uint64_t* lo)
{
    unsigned __int128 v = sumsq_exact(x, k);
    *hi = (uint64_t)(v >> 64);
    *lo = (uint64_t)v;
}

/* Exposed for the pins: or_ratio_to_f32 with a 128-bit numerator in halves. */
float or_ratio_to_f32_parts(uint64_t num_hi, uint64_t num_lo, uint64_t den, int e2)
{
    unsigned __int128 num = ((unsigned __int128)num_hi << 64) | num_lo;
    return or_ratio_to_f32(num, den, e2);
}


/* ------------------------------------------------------------------------ */
/* AWQ scale search                                                          */
/* ------------------------------------------------------------------------ */

/* Step 14's smoothing vector for one ratio. */
void or_awq_scales(const float* a, const float* b, int64_t k, double alpha, float* s)
{
    for (int64_t j = 0; j < k; ++j)
        s[j] = (a[j] == 0.0f || b[j] == 0.0f)
                   ? 1.0f
                   : (float)exp(alpha * log((double)a[j]) - (1.0 - alpha) * log((double)b[j]));
}

/*
 * Steps 13-15.  x fp16 [t, k] (calibration tokens), w float32 [n, k].  Outputs:
 * err float64 [grid], *best, s_best float32 [k] (the smoothing vector of the
 * chosen ratio).  quant = 0 replaces the int4 round trip of W' by its plain
 * fp16 rounding (a lossless stand-in the tests use).
 */
int or_awq_search(const uint16_t* x, int64_t t, const float* w, int64_t n, int64_t k, int G, int grid, int quant,
                  double* err, int* best, float* s_best)
{
    if (t <= 0 || n <= 0 || k <= 0 || G <= 0 || k % G || grid <= 0)
        return OR_BAD;
    const int64_t ng = k / G;
    float* a = (float*)calloc((size_t)k, sizeof(float));
    float* b = (float*)calloc((size_t)k, sizeof(float));
    float* s = (float*)malloc((size_t)k * sizeof(float));
    float* ws = (float*)malloc((size_t)(n * k) * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)(n * k));
    uint8_t* z = (uint8_t*)malloc((size_t)(n * ng));
    uint16_t* sc = (uint16_t*)malloc((size_t)(n * ng) * sizeof(uint16_t));
    uint16_t* wd16 = (uint16_t*)malloc((size_t)(n * k) * sizeof(uint16_t));
    uint16_t* xs = (uint16_t*)malloc((size_t)(t * k) * sizeof(uint16_t));
    double* yref = (double*)malloc((size_t)(t * n) * sizeof(double));
    double* erow = (double*)malloc((size_t)n * sizeof(double));
    if (!a || !b || !s || !ws || !q || !z || !sc || !wd16 || !xs || !yref || !erow) {
        free(a); free(b); free(s); free(ws); free(q); free(z); free(sc); free(wd16); free(xs); free(yref);
        free(erow);
        return OR_BAD;
    }
    for (int64_t j = 0; j < k; ++j) {
        for (int64_t i = 0; i < t; ++i) {
            float v = fabsf(or_f16_to_f32(x[i * k + j]));
            if (v > a[j]) a[j] = v;
        }
        for (int64_t r = 0; r < n; ++r) {
            float v = fabsf(w[r * k + j]);
            if (v > b[j]) b[j] = v;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < t; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)or_f16_to_f32(x[i * k + j]) * (double)w[r * k + j];
            yref[i * n + r] = acc;
        }
    int bi = 0;
    for (int g = 0; g < grid; ++g) {
        or_awq_scales(a, b, k, (double)g / (double)grid, s);
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < n; ++r)
            for (int64_t j = 0; j < k; ++j)
                ws[r * k + j] = w[r * k + j] * s[j];
        if (quant) {
            or_awq_quantize(ws, n, k, G, q, z, sc);
            or_awq_dequant(q, z, sc, n, k, G, NULL, wd16);
        } else {
            for (int64_t e = 0; e < n * k; ++e)
                wd16[e] = or_f32_to_f16(ws[e]);
        }
        for (int64_t i = 0; i < t; ++i)
            for (int64_t j = 0; j < k; ++j)
                xs[i * k + j] = or_f32_to_f16(or_f16_to_f32(x[i * k + j]) / s[j]);
        /* squared error per output channel, then the channels summed in
           order: the total does not depend on the thread count */
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < n; ++r) {
            double er = 0.0;
            for (int64_t i = 0; i < t; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j)
                    acc += (double)or_f16_to_f32(xs[i * k + j]) * (double)or_f16_to_f32(wd16[r * k + j]);
                double d = (double)or_f16_to_f32(or_f64_to_f16(acc)) - yref[i * n + r];
                er += d * d;
            }
            erow[r] = er;
        }
        double e2 = 0.0;
        for (int64_t r = 0; r < n; ++r)
            e2 += erow[r];
        err[g] = e2;
        if (e2 < err[bi])
            bi = g;
    }
    or_awq_scales(a, b, k, (double)bi / (double)grid, s_best);
    *best = bi;
    free(a); free(b); free(s); free(ws); free(q); free(z); free(sc); free(wd16); free(xs); free(yref); free(erow);
    return OR_OK;
}
