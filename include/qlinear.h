/*
 * qlinear.h -- C ABI of libqlinear, the quantized linear layer for MI355X
 * (gfx950 / CDNA4).
 *
 * Two paths of LLM inference:
 *
 *   W4A16 (AWQ-style weight-only int4).  LMDeploy engineering walkthrough
 *   (zwxr.cn/news/301173), section 2: weights quantised per group along the
 *   input dimension with their own scale, an asymmetric zero point from each
 *   group's min/max, group sizes 32/64/128 (CLI default 128); AUQ dual-process
 *   page (bjbfmj.com/news/39067), sections 3.3 and 5.4: the tensors qweight,
 *   scales, zeros and the dequantisation "int4 times scale with zero point".
 *
 *   W8A8 (SmoothQuant).  LMDeploy W8A8 guide (m.nxbn.cn/news/126471),
 *   "step 2: weight smoothing" (alpha = 0.5, norm weight divided by s, linear
 *   weight multiplied by s along its input dimension) and "inference kernels:
 *   QRMSNorm and QLinear" (RMSNorm fused with per-token dynamic int8
 *   quantisation; per-channel int8 weights with an fp32 scale; 8-bit GEMM with
 *   an int32 accumulator; output = acc * rms_scale * linear_scale in fp16).
 *
 * Conventions for every entry point
 *   - fp16 tensors are passed as uint16_t bit patterns (IEEE binary16).
 *   - All matrices are dense row-major.  x is [m, k]; weights are [n, k]
 *     (n output channels, k input channels: the torch Linear layout); y is
 *     [m, n].
 *   - "host" pointers are ordinary CPU memory; the call is synchronous.
 *     "device" pointers are HIP device memory of the current device; the call
 *     only enqueues work on `stream` (a hipStream_t, NULL = the null stream)
 *     and returns without synchronising.  Execution faults surface at the
 *     caller's next synchronisation.
 *   - The caller owns every buffer.  The device entry points never allocate
 *     or free memory and keep no state between calls, except a thread-local
 *     error message and per-device attributes queried once (compute units,
 *     LDS size).  The host helpers (ql_awq_pack, ql_awq_search, ...) use
 *     temporary host memory of their own while they run.
 *   - Return value: QL_OK (0) or a negative QL_ERR_* code.  On any error
 *     nothing is launched and no output is written; ql_last_error() gives a
 *     human-readable reason on the calling thread.
 *   - m == 0 or n == 0 is an empty problem: QL_OK, nothing launched.
 *     Negative sizes are QL_ERR_SHAPE.
 *   - Device pointers must be 16-byte aligned (128-bit loads and stores), or
 *     QL_ERR_ALIGN.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QL_OK 0
#define QL_ERR_NULL (-1)        /* a required pointer is NULL */
#define QL_ERR_SHAPE (-2)       /* negative size, k not a multiple of 8 or of group, ... */
#define QL_ERR_GROUP (-3)       /* group not in {32, 64, 128} */
#define QL_ERR_ALIGN (-4)       /* device pointer not 16-byte aligned */
#define QL_ERR_WORKSPACE (-5)   /* workspace missing or smaller than required */
#define QL_ERR_UNSUPPORTED (-6) /* shape or path the kernels do not cover */
#define QL_ERR_VALUE (-7)       /* non-finite input, or a scale outside fp16 range */
#define QL_ERR_HIP (-8)         /* a HIP runtime call or launch failed */

/* W4A16 kernel selection for ql_w4a16_gemm_path */
#define QL_PATH_AUTO 0          /* by m: decode path for m <= 64, MFMA GEMM above */
#define QL_PATH_DECODE 1        /* split-K GEMV path, m <= 64 */
#define QL_PATH_GEMM 2          /* LDS-tiled fp16 MFMA GEMM, any m */

/* ------------------------------------------------------------------------ */
/* W4A16                                                                      */
/* ------------------------------------------------------------------------ */

/*
 * ql_awq_pack (host).  Group-wise asymmetric uint4 quantisation of a float32
 * weight w [n, k] and packing, as in the LMDeploy walkthrough, section 2
 * (per-group min/max, asymmetric zero point) with the tensor names of the AUQ
 * page, section 5.4.  Per row r and group g (columns [g*group, (g+1)*group)):
 *   lo = min(0, min w), hi = max(0, max w)
 *   s  = fp16 value of max((hi - lo) / 15, 2^-14) rounded toward +infinity
 *   z  = clamp(rint(-lo / s), 0, 15)
 *   q  = clamp(rint(w / s) + z, 0, 15)           (rint: nearest, ties to even)
 * Rounding the scale up guarantees |w - (q - z) * s| <= s / 2.
 * Outputs
 *   qweight int32 [n, k/8]: word j of row r holds q[r, 8j + i] in bits
 *                           [4i, 4i + 4), i = 0..7
 *   scales  fp16  [n, k/group]
 *   qzeros  int32 [n, ceil(k/group/8)]: zero point of group g in bits
 *                           [4(g%8), 4(g%8) + 4) of word g/8; pad nibbles 0
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (n < 0, k <= 0, k % group != 0),
 * QL_ERR_GROUP, QL_ERR_VALUE (non-finite weight, or (hi - lo) / 15 above the
 * largest fp16).
 */
int ql_awq_pack(const float* w, int64_t n, int64_t k, int group,
                int32_t* qweight, uint16_t* scales, int32_t* qzeros);

/*
 * Bytes of device workspace ql_w4a16_gemm needs for this shape (0 if none),
 * enough for every kernel path ql_w4a16_gemm_path may take.  The workspace
 * holds what split-K launches exchange: the decode kernels (m <= 64) split K
 * when their column blocks alone would leave CUs idle, and so does the MFMA
 * GEMM when its tiles would.  Launches split in two meet in exchange slots;
 * launches split further use per-tile arrival counters and fp32 partial sums.
 */
size_t ql_w4a16_workspace_bytes(int64_t m, int64_t n, int64_t k, int group);

/* Leading bytes of a W4A16 workspace that must be zero before its first use
 * and that every completed call leaves zero. */
#define QL_W4A16_WS_ZERO_BYTES (32768u + (4u << 20))

/*
 * ql_w4a16_gemm (device).  The W4A16 linear layer of the LMDeploy
 * walkthrough, section 2 (int4 weights in groups along k, each group with its
 * own fp16 scale and an asymmetric uint4 zero point), dequantised as the AUQ
 * page, section 3.3, states it (int4 value times scale, with the zero point):
 *   y[m, n] = sum_c x[m, c] * (q[n, c] - z[n, g]) * s[n, g],  g = c / group
 * with fp32 accumulation and y rounded once to fp16.  The arithmetic of the
 * weight factor depends on the kernel that runs:
 *   - group 32 or 64, and any group with m > 64: each weight is formed as
 *     w16 = fp16((q - z) * s), one rounding of the exact product (the value
 *     ql_w4a16_dequant returns), and the exact fp16 x fp16 products x * w16
 *     are summed in fp32.
 *   - group 128 with m <= 64 (the decode kernels): the exact integers q - z
 *     multiply the activations (exact products), each 32-term partial sum
 *     within one group is formed in fp32 by the matrix cores, then multiplied
 *     by s and added to the fp32 accumulator in one fused multiply-add; w16
 *     is never formed.  Per
 *     term this differs from the first form only by w16's rounding, at most
 *     2^-11 of the weight, and a single nonzero activation (x = e_c) still
 *     gives y = w16[:, c] bit for bit, since (q - z) * s is exact in fp32.
 * The summation order is unspecified but fixed: repeating a call on the same
 * inputs gives the same bits.  Packed weights are streamed from HBM once per
 * call for m <= 64 and dequantised in registers.
 *   x        fp16 [m, k]            (device)
 *   qweight, scales, qzeros         as written by ql_awq_pack (device)
 *   y        fp16 [m, n]            (device, written)
 *   workspace, workspace_bytes      device scratch of at least
 *            ql_w4a16_workspace_bytes(m, n, k, group) bytes: a fixed region
 *            of 32 KiB + 4 MiB (QL_W4A16_WS_ZERO_BYTES: split-K arrival
 *            counters, then the slots in which two-slice launches exchange
 *            their partial sums) followed by fp32 partial sums.  Its first
 *            use must find the fixed region zero-filled; every completed call
 *            leaves it zero again, so one zeroed buffer serves any number of
 *            calls of any shape on one stream.  Calls that may run
 *            concurrently need separate workspaces.  May be NULL when the
 *            size is 0.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_GROUP, QL_ERR_ALIGN,
 * QL_ERR_WORKSPACE, QL_ERR_HIP.
 */
int ql_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                  const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k,
                  int group, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ql_w4a16_gemm_noalloc (device).  ql_w4a16_gemm for callers that cannot
 * allocate device memory -- code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc: the same kernels, results
 * bit-identical to ql_w4a16_gemm, with the split-K workspace taken from a
 * scratch array the library holds in device memory instead of an argument.
 *   Arguments as ql_w4a16_gemm, without the workspace.
 *   Scratch: 32 MiB per device (the QL_W4A16_WS_ZERO_BYTES region of
 *   counters and exchange slots, then partial sums), placed when the
 *   library's code loads on that device and held until the process ends;
 *   the first call on a device clears that region with a small kernel on
 *   `stream`, and every completed call leaves it zero.
 *   The call itself allocates nothing (no hipMalloc, no library allocator).
 *   Every call on a device shares that device's scratch: calls that may
 *   overlap on one device (other streams, other threads) race and must be
 *   serialised by the caller.
 * Errors: as ql_w4a16_gemm; QL_ERR_WORKSPACE when the shape needs more
 * split-K scratch than the array holds (ql_w4a16_workspace_bytes > 32 MiB);
 * QL_ERR_HIP if the scratch array's address cannot be obtained.
 */
int ql_w4a16_gemm_noalloc(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                          const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k, int group,
                          void* stream);

/* As ql_w4a16_gemm with an explicit kernel choice (QL_PATH_*), for tests and
 * tuning.  QL_PATH_DECODE with m > 64 is QL_ERR_UNSUPPORTED. */
int ql_w4a16_gemm_path(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                       const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k,
                       int group, void* workspace, size_t workspace_bytes, void* stream,
                       int path);

/*
 * ql_w4a16_dequant (device).  Runs the same device dequantisation routine the
 * GEMM kernels use and writes its results out.
 *   w16   fp16 [n, k]  dequantised weights (device, written)
 *   q_u8  uint8 [n, k] unpacked codes (device, written; may be NULL)
 * Errors as ql_w4a16_gemm (no workspace).
 */
int ql_w4a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                     uint16_t* w16, uint8_t* q_u8, int64_t n, int64_t k, int group,
                     void* stream);

/*
 * ql_awq_search (host, using the device).  Activation-aware choice of the
 * per-input-channel smoothing applied before the int4 quantisation: AWQ
 * picks the scales from sampled activations so that the product's error, not
 * the weights', is smallest (LMDeploy walkthrough, section 2), and the
 * smoothing coefficient is act_scales^alpha / w_scales^(1 - alpha) with the
 * ratio alpha searched per layer in calibration (LMDeploy W8A8 guide, source
 * analysis of the smoothing).  With a_j = max_t |x[t, j]|, b_j = max_r |w[r, j]|,
 * for alpha = i / grid, i = 0 .. grid-1:
 *   s_j  = exp(alpha ln a_j - (1 - alpha) ln b_j) in fp64, rounded to fp32
 *          (1 where a_j or b_j is 0)
 *   W'   = W diag(s), packed by ql_awq_pack;  x' = fp16(fp32(x) / s)
 *   y    = ql_w4a16_gemm(x', W') on the device (fp16)
 *   err_i = sum over (t, r) of (y - x w^T)^2, the reference in fp64
 * and the chosen ratio is the first i with the smallest err_i.
 *   x        fp16 [t, k] calibration tokens          (host)
 *   w        float32 [n, k]                          (host)
 *   grid     number of ratios, 1 .. 1000
 *   workspace, workspace_bytes   device scratch of at least
 *            ql_awq_search_workspace_bytes(t, n, k, group) bytes, 16-byte
 *            aligned, zero-filled before its first use (it holds the GEMM's
 *            split-K counters, which every call leaves zero)
 *   stream   hipStream_t (NULL = default); the call synchronises it
 *   err      float64 [grid]    (host, written)
 *   best     chosen index      (host, written)
 *   s_best   float32 [k]       (host, written): the chosen smoothing vector;
 *            the layer then computes (x / s_best) W'^T
 *   qweight, scales, qzeros   (host, written; all NULL to skip): the chosen
 *            W' packed as by ql_awq_pack
 * Errors: QL_ERR_NULL, QL_ERR_GROUP, QL_ERR_SHAPE (t, n, k <= 0, k % group,
 * grid out of range), QL_ERR_UNSUPPORTED (t*k or t*n >= 2^30, n*k >= 2^32),
 * QL_ERR_WORKSPACE, QL_ERR_ALIGN, QL_ERR_VALUE (non-finite weight, or a
 * smoothed group whose scale leaves fp16), QL_ERR_HIP, and those of
 * ql_w4a16_gemm.
 */
size_t ql_awq_search_workspace_bytes(int64_t t, int64_t n, int64_t k, int group);
int ql_awq_search(const uint16_t* x, int64_t t, const float* w, int64_t n, int64_t k, int group, int grid,
                  void* workspace, size_t workspace_bytes, void* stream, double* err, int* best,
                  float* s_best, int32_t* qweight, uint16_t* scales, int32_t* qzeros);

/* ------------------------------------------------------------------------ */
/* W8A8 (SmoothQuant)                                                        */
/* ------------------------------------------------------------------------ */

/*
 * ql_smooth (host).  SmoothQuant smoothing with alpha = 0.5 (LMDeploy W8A8
 * guide, "step 2: weight smoothing").  For each input channel j:
 *   a_j = max over rows of |x[:, j]|,  b_j = max over n of |w[:, j]|
 *   s_j = sqrt(a_j) / sqrt(b_j)   (s_j = 1 where a_j, b_j or gamma_j is 0)
 *   gamma_smoothed_j = fp16(gamma_j / s_j),  w_smoothed[:, j] = w[:, j] * s_j
 *   x      fp16 [rows, k]  activations whose column maxima define a_j (host)
 *   gamma  fp16 [k]        RMSNorm weight feeding the linear (host)
 *   w      float32 [n, k]  linear weight (host)
 *   s float32 [k], gamma_smoothed fp16 [k], w_smoothed float32 [n, k] (host, written)
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_VALUE (non-finite input).
 */
int ql_smooth(const uint16_t* x, int64_t rows, const uint16_t* gamma, const float* w,
              int64_t n, int64_t k, float* s, uint16_t* gamma_smoothed, float* w_smoothed);

/*
 * ql_w8a8_quant_weight (host).  Per-output-channel symmetric int8 weights
 * (LMDeploy W8A8 guide, QLinear.from_float / per_channel_quant):
 *   w_scale[r] = max_j |w[r, j]| / 127
 *   wq[r, j]   = clamp(rint(w[r, j] / w_scale[r]), -127, 127)  (0 for a zero row)
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_VALUE (non-finite weight).
 */
int ql_w8a8_quant_weight(const float* w, int64_t n, int64_t k, int8_t* wq, float* w_scale);

/*
 * ql_w8a8_quant_rmsnorm (device).  QRMSNorm: RMSNorm fused with per-token
 * dynamic int8 quantisation (LMDeploy W8A8 guide, "inference kernels":
 * rms_norm_dynamic_quant, per-token scale = absmax / 127).  Per token i, in
 * fp32:
 *   ms  = sum_j x[i,j]^2 / k, computed exactly and rounded once to fp32
 *   r   = 1 / sqrt(ms + eps)
 *   y_j = (x[i,j] * r) * gamma[j]
 *   x_scale[i] = max_j |y_j| / 127
 *   xq[i,j]    = clamp(rint(y_j / x_scale[i]), -127, 127)  (0 for x_scale 0)
 * Divisions and the square root are correctly rounded, so results are
 * bit-identical to any exact implementation of these definitions.
 *   x fp16 [m, k], gamma fp16 [k] (device); xq int8 [m, k], x_scale float32 [m]
 *   (device, written).  k <= 65536.  Inputs must be finite.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_UNSUPPORTED,
 * QL_ERR_HIP.
 */
int ql_w8a8_quant_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps,
                          int8_t* xq, float* x_scale, int64_t m, int64_t k, void* stream);

/*
 * ql_w8a8_gemm (device).  QLinear forward on a quantised activation
 * (LMDeploy W8A8 guide, matmul_kernel_dynamic_quant): int8 x int8 products
 * accumulated exactly in int32, then y = fp16((float)acc * x_scale[i] *
 * w_scale[j]).
 *   xq int8 [m, k], x_scale float32 [m], wq int8 [n, k], w_scale float32 [n]
 *   (device); y fp16 [m, n] (device, written).
 *   k <= 131072 keeps |acc| <= 127 * 127 * k below 2^31.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_UNSUPPORTED, QL_ERR_HIP.
 */
int ql_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                 uint16_t* y, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * ql_w8a8_add_quant_rmsnorm (device).  QRMSNorm with the residual add fused in
 * front (LMDeploy W8A8 guide, "inference kernels": the RMSNorm dynamic-quant
 * kernel's residual fusion).  Per element h = fp16(x + residual), the exact
 * sum rounded once; h is written to h_out (the updated residual stream), then
 * xq / x_scale are QRMSNorm of h exactly as ql_w8a8_quant_rmsnorm defines it.
 *   x, residual fp16 [m, k], gamma fp16 [k] (device); h_out fp16 [m, k], xq
 *   int8 [m, k], x_scale float32 [m] (device, written).  h_out may be x or
 *   residual (in-place update); it must not overlap them otherwise.
 *   k <= 65536.  Inputs must be finite.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_VALUE, QL_ERR_ALIGN,
 * QL_ERR_UNSUPPORTED, QL_ERR_HIP.
 */
int ql_w8a8_add_quant_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                              float eps, uint16_t* h_out, int8_t* xq, float* x_scale,
                              int64_t m, int64_t k, void* stream);

/*
 * ql_w8a8_quant_per_token (device).  Per-token dynamic int8 quantisation of a
 * plain activation, for a QLinear whose input does not come from QRMSNorm
 * (LMDeploy W8A8 guide, "inference kernels": per_token_quant_int8, scale =
 * absmax / Q_MAX).  Per token i, in fp32:
 *   x_scale[i] = max_j |x[i,j]| / 127
 *   xq[i,j]    = clamp(rint(x[i,j] / x_scale[i]), -127, 127)  (0 for x_scale 0)
 * both correctly rounded divisions.
 *   x fp16 [m, k] (device); xq int8 [m, k], x_scale float32 [m] (device,
 *   written).  k <= 65536.  Inputs must be finite.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_UNSUPPORTED,
 * QL_ERR_HIP.
 */
int ql_w8a8_quant_per_token(const uint16_t* x, int8_t* xq, float* x_scale,
                            int64_t m, int64_t k, void* stream);

/*
 * ql_w8a8_gemm_ex (device).  ql_w8a8_gemm with the optional bias and residual
 * of the epilogue (LMDeploy W8A8 guide, "inference kernels": the int8 GEMM's
 * residual and bias fusion after the rms_scale * linear_scale dequantisation):
 *   y = fp16(fp32(fp32(fp32(fp32(acc * x_scale[i]) * w_scale[j]) + bias[j])
 *            + residual[i,j]))
 * each fp32 operation rounded on its own, a term skipped (not added as 0)
 * when its pointer is NULL.
 *   bias fp16 [n] or NULL, residual fp16 [m, n] or NULL (device); y fp16
 *   [m, n] (device, written) may be residual itself (in-place add); other
 *   arguments as ql_w8a8_gemm.
 * Errors: as ql_w8a8_gemm.
 */
int ql_w8a8_gemm_ex(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                    const uint16_t* bias, const uint16_t* residual, uint16_t* y,
                    int64_t m, int64_t n, int64_t k, void* stream);

/* ------------------------------------------------------------------------ */
/* W8A8 with FP8 E4M3 (float8_e4m3fn) codes                                    */
/* ------------------------------------------------------------------------ */
/*
 * The LMDeploy W8A8 guide's second 8-bit type (--quant-dtype fp8 is
 * float8_e4m3fn; Q_MAX is the type's largest finite value, 448; the codes are
 * a cast, not rint + clamp; the GEMM accumulates in fp32).  Codes are OCP FP8
 * E4M3 bytes: sign, 4 exponent bits with bias 7, 3 fraction bits, no
 * infinities, S.1111.111 is NaN.  The cast rounds to nearest, ties to even.
 */

/*
 * ql_fp8_quant_weight (host, synchronous).  Per output channel n:
 *   w_scale[n] = max_j |w[n,j]| / 448,  wq[n,j] = e4m3(w[n,j] / w_scale[n])
 * (an all-zero row gets scale 0 and codes 0).  w fp32 [n, k] (host); wq uint8
 * [n, k] and w_scale float32 [n] (host, written).
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_VALUE (non-finite weight).
 */
int ql_fp8_quant_weight(const float* w, int64_t n, int64_t k, uint8_t* wq, float* w_scale);

/*
 * ql_fp8_quant_rmsnorm (device).  QRMSNorm with FP8 codes: y as in
 * ql_w8a8_quant_rmsnorm, then x_scale[i] = max_j |y_j| / 448 and
 * xq[i,j] = e4m3(y_j / x_scale[i]) (correctly rounded fp32 divisions).
 *   x fp16 [m, k], gamma fp16 [k] (device); xq uint8 [m, k], x_scale float32
 *   [m] (device, written).  k <= 65536.  Inputs must be finite.
 * Errors: as ql_w8a8_quant_rmsnorm.
 */
int ql_fp8_quant_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps,
                         uint8_t* xq, float* x_scale, int64_t m, int64_t k, void* stream);

/*
 * ql_fp8_quant_per_token (device).  Per-token FP8 quantisation of a plain
 * activation: x_scale[i] = max_j |x[i,j]| / 448, xq[i,j] = e4m3(x[i,j] / x_scale[i]).
 * Arguments and errors as ql_w8a8_quant_per_token (xq uint8 bytes).
 */
int ql_fp8_quant_per_token(const uint16_t* x, uint8_t* xq, float* x_scale,
                           int64_t m, int64_t k, void* stream);

/*
 * ql_fp8_gemm (device).  FP8 QLinear: acc[i,j] = sum_k e4m3(xq[i,k]) *
 * e4m3(wq[j,k]), products exact and summed in fp32 by the matrix cores (order
 * unspecified), then the epilogue of ql_w8a8_gemm_ex:
 *   y = fp16(fp32(fp32(fp32(fp32(acc * x_scale[i]) * w_scale[j]) + bias[j]) + residual[i,j]))
 *   xq uint8 [m, k], x_scale float32 [m], wq uint8 [n, k], w_scale float32
 *   [n], bias fp16 [n] or NULL, residual fp16 [m, n] or NULL (device); y fp16
 *   [m, n] (device, written; may be residual).  k % 64 == 0.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_UNSUPPORTED
 * (k % 64, k above 131072, or xq or wq of 4 GiB or more), QL_ERR_HIP.
 */
int ql_fp8_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                const uint16_t* bias, const uint16_t* residual, uint16_t* y,
                int64_t m, int64_t n, int64_t k, void* stream);

/* ------------------------------------------------------------------------ */
/* KV cache INT8                                                              */
/* ------------------------------------------------------------------------ */
/*
 * ql_kv_quant_int8 (device).  KV-cache group quantisation between FP16 and
 * INT8 (FastLLM architecture page, section 5.2: groups of 128).  Per group of
 * `group` consecutive values (a head's vector of the K or V cache at 128):
 *   scale[g] = max |x| / 127,  q = clamp(rint(x / scale[g]), -127, 127)
 * (correctly rounded fp32 divisions; a zero group gets scale 0 and codes 0).
 *   x fp16 [groups * group] (device); q int8 [groups * group], scale float32
 *   [groups] (device, written).  group in {32, 64, 128}.  Inputs finite.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_GROUP, QL_ERR_ALIGN,
 * QL_ERR_UNSUPPORTED, QL_ERR_HIP.
 */
int ql_kv_quant_int8(const uint16_t* x, int8_t* q, float* scale, int64_t groups, int group, void* stream);

/*
 * ql_kv_dequant_int8 (device).  out = fp16(fp32(q * scale[g])): the fp32
 * product, cast to fp16 (nearest, ties to even).
 *   q int8 [groups * group], scale float32 [groups] (device); out fp16
 *   [groups * group] (device, written).  Errors: as ql_kv_quant_int8.
 */
int ql_kv_dequant_int8(const int8_t* q, const float* scale, uint16_t* out, int64_t groups, int group,
                       void* stream);

/* ql_w8a8_gemm_i32 (device).  The same int8 MFMA main loop writing the raw
 * int32 accumulator acc [m, n] instead of the fp16 epilogue. */
int ql_w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc,
                     int64_t m, int64_t n, int64_t k, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                                */
/* ------------------------------------------------------------------------ */

/* Static name of a status code ("QL_OK", "QL_ERR_SHAPE", ...). */
const char* ql_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* ql_last_error(void);
/* Library ABI version (major * 10000 + minor * 100 + patch). */
int ql_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
