// W4A16 kernels for gfx950 and their C-ABI entry points.
//
//   w4a16_dequant_kernel  -- writes the shared dequantisation routine's output
//   w4a16_decode_kernel   -- m <= 32: split-K GEMV on MFMA, weights streamed
//                            from HBM once, dequantised in registers
//   w4a16_gemm_kernel     -- any m: LDS-tiled fp16 MFMA GEMM
//
// Weight format (LMDeploy walkthrough, section 2; AUQ page, section 5.4):
// qweight int32 [n, k/8] with code i of a word at bits [4i, 4i+4), fp16 scales
// [n, k/group], uint4 zero points packed eight to an int32 [n, ceil(k/group/8)].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "dequant.hpp"
#include "ql_common.hpp"

using ql::f4_t;
using ql::h2_t;
using ql::h8_t;

namespace {

// MFMA 16x16x32 fp16 -> fp32.  Lane l supplies A[l%16][8(l/16) .. +7] and
// B[8(l/16) .. +7][l%16]; it receives D[4(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ f4_t mfma16x16x32(h8_t a, h8_t b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ---------------------------------------------------------------------------
// dequant export: one thread per packed word
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4a16_dequant_kernel(const uint32_t* __restrict__ qw,
                                                            const uint16_t* __restrict__ sc,
                                                            const uint32_t* __restrict__ qz,
                                                            uint16_t* __restrict__ w16,
                                                            uint8_t* __restrict__ q8, int N, int K, int G)
{
    const int KW = K / 8, NG = K / G, ZW = (NG + 7) / 8;
    const int64_t total = (int64_t)N * KW;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / KW), j = (int)(i - (int64_t)n * KW);
        const int g = (8 * j) / G;
        const uint32_t w = qw[i];
        h2_t o[4];
        ql::dequant_word(w, ql::zero_bias(ql::zero_of(qz + (int64_t)n * ZW, g)),
                         ql::scale2(sc[(int64_t)n * NG + g]), o);
        // back to natural order: (0,4)(1,5)(2,6)(3,7) -> 0..7
        const uint32_t a = ql::h2u(o[0]), b = ql::h2u(o[1]), c = ql::h2u(o[2]), d = ql::h2u(o[3]);
        uint4 u;
        u.x = (a & 0xFFFFu) | (b << 16);
        u.y = (c & 0xFFFFu) | (d << 16);
        u.z = (a >> 16) | (b & 0xFFFF0000u);
        u.w = (c >> 16) | (d & 0xFFFF0000u);
        *reinterpret_cast<uint4*>(w16 + i * 8) = u;
        if (q8) {
            uint2 cq;
            cq.x = (w & 0xFu) | ((w >> 4) & 0xFu) << 8 | ((w >> 8) & 0xFu) << 16 | ((w >> 12) & 0xFu) << 24;
            cq.y = ((w >> 16) & 0xFu) | ((w >> 20) & 0xFu) << 8 | ((w >> 24) & 0xFu) << 16 | (w >> 28) << 24;
            *reinterpret_cast<uint2*>(q8 + i * 8) = cq;
        }
    }
}

// ---------------------------------------------------------------------------
// decode: m <= MT (16 or 32)
//
// Workgroup = NT waves; wave w owns 16 output channels; the workgroup covers a
// K slice of NB blocks of 256.  In a block, lane l (row l%16, quarter
// q = l/16) loads two 16-byte pieces of its row: words [4q, 4q+4) and
// [16+4q, 16+4q+4), so 4 lanes read 64 contiguous bytes per row per load.
// Word j of piece i feeds MFMA 4i+j; the matching activations are chunk
// 16i + 4q + j of the block, staged once per workgroup in LDS in the
// dequantiser's element order.  All NB blocks are requested before any is
// consumed.  Slices are combined in fixed order by the last workgroup to
// finish a column block (deterministic split-K).
// ---------------------------------------------------------------------------
constexpr int kDecodeNT = 4;

template <int MT, int NT, int NB>
__global__ __launch_bounds__(64 * NT) void w4a16_decode_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int M, int N, int K, int G)
{
    constexpr int KS = NB * 256;        // k per slice
    constexpr int CH = KS / 8;          // 8-element chunks per slice
    constexpr int RS = CH + 1;          // LDS row stride in uint4 (16-byte pad)
    __shared__ uint4 xs[MT * RS];
    __shared__ int s_last;

    const int S = gridDim.y;
    const int k0 = blockIdx.y * KS;
    const int kend = min(K, k0 + KS);
    const int nch = (kend - k0) >> 3;

    // activations of this slice -> LDS (rows < M only; chunks past K are zero)
    for (int idx = threadIdx.x; idx < M * CH; idx += 64 * NT) {
        const int m = idx / CH, c = idx - m * CH;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (c < nch)
            v = ql::permute_x8(*reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + 8 * c));
        xs[m * RS + c] = v;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int n = (blockIdx.x * NT + wave) * 16 + r16;
    const bool nok = n < N;
    const int KW = K >> 3, NG = K / G, ZW = (NG + 7) >> 3;
    const uint32_t* qrow = qw + (int64_t)(nok ? n : 0) * KW;
    const uint16_t* srow = sc + (int64_t)(nok ? n : 0) * NG;
    const uint32_t* zrow = qz + (int64_t)(nok ? n : 0) * ZW;

    uint4 wv[NB][2];
    uint32_t sv[NB][2], zv[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kk = k0 + b * 256 + i * 128 + 32 * q;
            const bool ok = nok && kk < kend;
            wv[b][i] = ok ? *reinterpret_cast<const uint4*>(qrow + (kk >> 3)) : make_uint4(0u, 0u, 0u, 0u);
            const int g = kk / G;
            sv[b][i] = ok ? srow[g] : 0u;
            zv[b][i] = ok ? ql::zero_of(zrow, g) : 0u;
        }
    __syncthreads();

    f4_t acc[MT / 16];
#pragma unroll
    for (int t = 0; t < MT / 16; ++t)
        acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const h2_t zb = ql::zero_bias(zv[b][i]), s2 = ql::scale2(sv[b][i]);
            const uint32_t words[4] = {wv[b][i].x, wv[b][i].y, wv[b][i].z, wv[b][i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8_t bw = ql::dequant_word8(words[j], zb, s2);
                const int c = b * 32 + i * 16 + 4 * q + j;
#pragma unroll
                for (int t = 0; t < MT / 16; ++t) {
                    const int m = t * 16 + r16;
                    h8_t a = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
                    if (m < M)
                        a = __builtin_bit_cast(h8_t, xs[m * RS + c]);
                    acc[t] = mfma16x16x32(a, bw, acc[t]);
                }
            }
        }

    if (S == 1) {
#pragma unroll
        for (int t = 0; t < MT / 16; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t * 16 + 4 * q + r;
                if (m < M && nok)
                    y[(int64_t)m * N + n] = f32_to_f16_bits(acc[t][r]);
            }
        return;
    }

    // split-K: publish this slice's partial sums, the last arrival reduces
#pragma unroll
    for (int t = 0; t < MT / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = t * 16 + 4 * q + r;
            if (m < M && nok)
                part[((int64_t)blockIdx.y * M + m) * N + n] = acc[t][r];
        }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&cnt[blockIdx.x], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    const int nb0 = blockIdx.x * NT * 16;
    for (int idx = threadIdx.x; idx < M * NT * 16; idx += 64 * NT) {
        const int m = idx / (NT * 16), nn = nb0 + idx - m * (NT * 16);
        if (nn < N) {
            float s = 0.f;
            for (int sl = 0; sl < S; ++sl)
                s += __builtin_nontemporal_load(&part[((int64_t)sl * M + m) * N + nn]);
            y[(int64_t)m * N + nn] = f32_to_f16_bits(s);
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// GEMM: block tile 128 (m) x 128 (n), 4 waves as 2 x 2, wave tile 64 x 64.
// K advances in super-steps of 128.  The activation tile goes through LDS in
// the dequantiser's element order; each wave streams its own 64 weight rows
// straight into registers (one 16-byte piece per lane and 16-row tile per
// super-step) and dequantises them there.
// ---------------------------------------------------------------------------
constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 128;

__global__ __launch_bounds__(256) void w4a16_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ sc,
                                                         const uint32_t* __restrict__ qz,
                                                         uint16_t* __restrict__ y, int M, int N, int K, int G)
{
    constexpr int CH = kGemmBK / 8;      // 16 chunks per row per super-step
    constexpr int RS = CH + 1;           // padded LDS row stride (uint4)
    __shared__ uint4 as[kGemmBM * RS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, r16 = lane & 15;
    const int m0 = blockIdx.y * kGemmBM, n0 = blockIdx.x * kGemmBN;
    const int KW = K >> 3, NG = K / G, ZW = (NG + 7) >> 3;

    int nrow[4];
    bool nok[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int n = n0 + wn * 64 + t * 16 + r16;
        nok[t] = n < N;
        nrow[t] = nok[t] ? n : 0;
    }

    f4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < K; kb += kGemmBK) {
        const int nch = min(CH, (K - kb) >> 3);
        // weights of this super-step (issued first: the longest latency)
        uint4 wv[4];
        uint32_t sv[4], zv[4];
        const int kk = kb + 32 * q;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool ok = nok[t] && kk < K;
            wv[t] = ok ? *reinterpret_cast<const uint4*>(qw + (int64_t)nrow[t] * KW + (kk >> 3))
                       : make_uint4(0u, 0u, 0u, 0u);
            const int g = kk / G;
            sv[t] = ok ? sc[(int64_t)nrow[t] * NG + g] : 0u;
            zv[t] = ok ? ql::zero_of(qz + (int64_t)nrow[t] * ZW, g) : 0u;
        }
        // activation tile -> LDS
        __syncthreads();
        for (int idx = threadIdx.x; idx < kGemmBM * CH; idx += 256) {
            const int r = idx / CH, c = idx - r * CH;
            const int m = m0 + r;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && c < nch)
                v = ql::permute_x8(*reinterpret_cast<const uint4*>(x + (int64_t)m * K + kb + 8 * c));
            as[r * RS + c] = v;
        }
        __syncthreads();

#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const h2_t zb = ql::zero_bias(zv[t]), s2 = ql::scale2(sv[t]);
            const uint32_t words[4] = {wv[t].x, wv[t].y, wv[t].z, wv[t].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8_t bw = ql::dequant_word8(words[j], zb, s2);
                const int c = 4 * q + j;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const h8_t a = __builtin_bit_cast(h8_t, as[(wm * 64 + i * 16 + r16) * RS + c]);
                    acc[i][t] = mfma16x16x32(a, bw, acc[i][t]);
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int n = n0 + wn * 64 + t * 16 + r16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + 4 * q + r;
                if (m < M && n < N)
                    y[(int64_t)m * N + n] = f32_to_f16_bits(acc[i][t][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct DecodePlan {
    int mt;     // 16 or 32
    int nb;     // 256-blocks per slice
    int slices; // split-K factor
    int nblk;   // column blocks
    size_t counter_bytes, part_offset, part_bytes;
};

DecodePlan decode_plan(int64_t m, int64_t n, int64_t k)
{
    DecodePlan p{};
    p.mt = m <= 16 ? 16 : 32;
    p.nb = p.mt == 16 ? 4 : 2;
    p.slices = (int)((k + p.nb * 256 - 1) / (p.nb * 256));
    p.nblk = (int)((n + kDecodeNT * 16 - 1) / (kDecodeNT * 16));
    p.counter_bytes = (size_t)p.nblk * sizeof(uint32_t);
    p.part_offset = (p.counter_bytes + 255) & ~(size_t)255;
    p.part_bytes = p.slices > 1 ? (size_t)p.slices * (size_t)m * (size_t)n * sizeof(float) : 0;
    return p;
}

size_t decode_workspace(const DecodePlan& p) { return p.slices > 1 ? p.part_offset + p.part_bytes : 0; }

int check_common(const void* qweight, const void* scales, const void* qzeros, int64_t n, int64_t k, int group,
                 const char* who)
{
    if (!qweight || !scales || !qzeros)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::valid_group(group))
        QL_FAIL(QL_ERR_GROUP, "%s: group %d not in {32, 64, 128}", who, group);
    if (n < 0 || k <= 0 || k % group)
        QL_FAIL(QL_ERR_SHAPE, "%s: n=%lld k=%lld group=%d", who, (long long)n, (long long)k, group);
    if (n > (1LL << 30) || k > (1LL << 30) || n * (k / 8) > (1LL << 40))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: n=%lld k=%lld too large", who, (long long)n, (long long)k);
    if (!ql::aligned16(qweight) || !ql::aligned16(scales) || !ql::aligned16(qzeros))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    return QL_OK;
}

int launch_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        QL_FAIL(QL_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return QL_OK;
}

template <int MT, int NB>
void launch_decode(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                   const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int g, hipStream_t st)
{
    uint32_t* cnt = p.slices > 1 ? static_cast<uint32_t*>(ws) : nullptr;
    float* part = p.slices > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset) : nullptr;
    hipLaunchKernelGGL((w4a16_decode_kernel<MT, kDecodeNT, NB>), dim3(p.nblk, p.slices), dim3(64 * kDecodeNT), 0,
                       st, x, qw, sc, qz, y, part, cnt, m, n, k, g);
}

}  // namespace

extern "C" size_t ql_w4a16_workspace_bytes(int64_t m, int64_t n, int64_t k, int group)
{
    (void)group;
    if (m <= 0 || n <= 0 || k <= 0 || m > 32)
        return 0;
    return decode_workspace(decode_plan(m, n, k));
}

extern "C" int ql_w4a16_gemm_path(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                                  const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k, int group,
                                  void* workspace, size_t workspace_bytes, void* stream, int path)
{
    ql::clear_error();
    const char* who = "ql_w4a16_gemm";
    if (int rc = check_common(qweight, scales, qzeros, n, k, group, who))
        return rc;
    if (m < 0)
        QL_FAIL(QL_ERR_SHAPE, "%s: m=%lld", who, (long long)m);
    if (m > (1LL << 30))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: m=%lld too large", who, (long long)m);
    if (path != QL_PATH_AUTO && path != QL_PATH_DECODE && path != QL_PATH_GEMM)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: unknown path %d", who, path);
    if (path == QL_PATH_AUTO)
        path = m <= 32 ? QL_PATH_DECODE : QL_PATH_GEMM;
    if (path == QL_PATH_DECODE && m > 32)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: decode path needs m <= 32 (m=%lld)", who, (long long)m);
    if (m == 0 || n == 0)
        return QL_OK;
    if (!x || !y)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(x) || !ql::aligned16(y))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const auto* xw = x;
    const auto* qw = reinterpret_cast<const uint32_t*>(qweight);
    const auto* qz = reinterpret_cast<const uint32_t*>(qzeros);
    const int mi = (int)m, ni = (int)n, ki = (int)k;

    if (path == QL_PATH_DECODE) {
        DecodePlan p = decode_plan(m, n, k);
        const size_t need = decode_workspace(p);
        if (need > 0 && (!workspace || workspace_bytes < need))
            QL_FAIL(QL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace ? workspace_bytes : (size_t)0);
        if (need > 0 && !ql::aligned16(workspace))
            QL_FAIL(QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
        if (p.mt == 16)
            launch_decode<16, 4>(p, xw, qw, scales, qz, y, workspace, mi, ni, ki, group, st);
        else
            launch_decode<32, 2>(p, xw, qw, scales, qz, y, workspace, mi, ni, ki, group, st);
        return launch_status(who);
    }
    dim3 grid((unsigned)((n + kGemmBN - 1) / kGemmBN), (unsigned)((m + kGemmBM - 1) / kGemmBM));
    hipLaunchKernelGGL(w4a16_gemm_kernel, grid, dim3(256), 0, st, xw, qw, scales, qz, y, mi, ni, ki, group);
    return launch_status(who);
}

extern "C" int ql_w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                             const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k, int group,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    return ql_w4a16_gemm_path(x, qweight, scales, qzeros, y, m, n, k, group, workspace, workspace_bytes, stream,
                              QL_PATH_AUTO);
}

extern "C" int ql_w4a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                                uint16_t* w16, uint8_t* q_u8, int64_t n, int64_t k, int group, void* stream)
{
    ql::clear_error();
    const char* who = "ql_w4a16_dequant";
    if (int rc = check_common(qweight, scales, qzeros, n, k, group, who))
        return rc;
    if (n == 0)
        return QL_OK;
    if (!w16)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(w16) || (q_u8 && !ql::aligned16(q_u8)))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    const int64_t words = n * (k / 8);
    const unsigned blocks = (unsigned)std::min<int64_t>((words + 255) / 256, 65536);
    hipLaunchKernelGGL(w4a16_dequant_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint32_t*>(qweight), scales, reinterpret_cast<const uint32_t*>(qzeros),
                       w16, q_u8, (int)n, (int)k, group);
    return launch_status(who);
}
