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
#include "lds_dma.hpp"
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
        const h2_t zb = ql::zero_bias(ql::zero_of(qz + (int64_t)n * ZW, g));
        const h2_t s2 = ql::scale2(sc[(int64_t)n * NG + g]);
        // Both in-register routines give the same natural-order values; even
        // words take the natural-order one (GEMM), odd words the (0,4)(1,5)
        // (2,6)(3,7) one (decode) put back in order, so the exported weights
        // check both.
        uint4 u;
        if ((j & 1) == 0) {
            u = __builtin_bit_cast(uint4, ql::dequant_word8_natural(w, zb, s2));
        } else {
            h2_t o[4];
            ql::dequant_word(w, zb, s2, o);
            const uint32_t a = ql::h2u(o[0]), b = ql::h2u(o[1]), c = ql::h2u(o[2]), d = ql::h2u(o[3]);
            u.x = (a & 0xFFFFu) | (b << 16);
            u.y = (c & 0xFFFFu) | (d << 16);
            u.z = (a >> 16) | (b & 0xFFFF0000u);
            u.w = (c >> 16) | (d & 0xFFFF0000u);
        }
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
// Workgroup = T waves; wave t owns 16 output channels, so a workgroup covers
// 16T channels and one K slice of KS (a multiple of 256).  The slice's
// activations (rows < m) are staged once in LDS, in the dequantiser's element
// order, and shared by the T waves.  Each wave then streams its 16 rows of the
// slice in blocks of 256 k through a P-deep register ring: as soon as block b
// is consumed its slot is refilled with block b + P, so every wave keeps about
// P x 2 KB of weights in flight.
//
// In a block, lane l (row l%16, quarter q = l/16) loads two 16-byte pieces of
// its row: words [4q, 4q+4) and [16+4q, 16+4q+4), so 4 lanes read 64
// contiguous bytes of a row per load.  Word j of piece i is the B operand of
// one MFMA directly; weights never pass through LDS.
//
// Weights, scales and zero points are read with buffer loads: a scalar
// resource per tensor and a 32-bit per-lane offset, so the per-block address
// arithmetic is one add or an immediate offset.  A read past a resource's end
// returns zero.  Lanes past N read row N-1 and their outputs are discarded;
// pieces past the slice end read finite words of the same tensor that meet
// zero activations (the staged slice is zero past K).  MFMA rows past m read
// a real activation row and are never stored.
//
// Split-K (S > 1 slices): each slice writes its fp32 partial tile with
// agent-scope stores, waits for them to complete, then bumps a per-column-block
// arrival counter; the last arrival reads the partials back with agent-scope
// loads and sums them in slice order (deterministic).  No cache-wide fence is
// needed because every cross-workgroup value travels through agent-scope
// accesses.
// ---------------------------------------------------------------------------
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}

template <int MT, int T, int P>
__global__ __launch_bounds__(64 * T) void w4a16_decode_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int M, int N, int K, int lg, int KS)
{
    // LDS: activations [min(M, MT)][RS] uint4, then per (row, group) of the
    // slice one word holding (fp16 scale | zero point << 16)
    extern __shared__ uint4 xs[];
    __shared__ int s_last;

    const int S = gridDim.y;
    const int k0 = blockIdx.y * KS;
    const int kend = min(K, k0 + KS);
    const int nch = (kend - k0) >> 3;
    const int nb = (kend - k0 + 255) >> 8;
    const int nbp = (nb + P - 1) / P * P;         // blocks streamed, padded to the ring
    const int RS = ((KS >> 8) + P - 1) / P * P * 32 + 1;   // padded slice + 16-byte pad
    const int mrows = M < MT ? M : MT;
    const int gs = KS >> lg;                      // groups per slice
    uint32_t* sz = reinterpret_cast<uint32_t*>(xs + mrows * RS);   // [16T][gs]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * T * 16;
    const int n = n0 + wave * 16 + r16;
    const bool nok = n < N;
    const int KW = K >> 3, NG = K >> lg, ZW = (NG + 7) >> 3;
    const uint32_t nr = (uint32_t)(nok ? n : N - 1);

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)KW * 4u);
    const uint32_t ow = nr * (uint32_t)KW * 4u + (uint32_t)(k0 + 32 * q) / 2u;   // block 0, piece 0
    auto load_block = [&](int b, uint4& w0, uint4& w1) {
        const uint32_t bw = ow + (uint32_t)b * 128u;
        w0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)bw, 0, 0));
        w1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(bw + 64u), 0, 0));
    };

    // 1. the first P weight blocks (unconditional: blocks past the slice
    // re-read block nb-1, so every wait in the stream has a static count)
    uint4 ring[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        load_block(p < nb ? p : nb - 1, ring[p][0], ring[p][1]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. scales and zero points of this workgroup's rows and slice -> LDS.
    //    Each thread issues four entries' loads (clamped, always in bounds)
    //    before using any, so the staging costs one memory latency, not four.
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc, (uint32_t)N * (uint32_t)NG * 2u);
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(qz, (uint32_t)N * (uint32_t)ZW * 4u);
        const int g0 = k0 >> lg;
        const int total = 16 * T * gs;
        for (int e0 = 0; e0 < total; e0 += 4 * 64 * T) {
            uint32_t sv[4], zw[4], gv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = min(e0 + u * 64 * T + (int)threadIdx.x, total - 1);
                const int rr = e / gs, gg = e - rr * gs;
                const uint32_t row = (uint32_t)min(n0 + rr, N - 1);
                const uint32_t g = (uint32_t)(g0 + gg);
                gv[u] = g;
                sv[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)((row * (uint32_t)NG + g) * 2u), 0, 0);
                zw[u] = __builtin_amdgcn_raw_buffer_load_b32(rz, (int)((row * (uint32_t)ZW + (g >> 3)) * 4u), 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * 64 * T + (int)threadIdx.x;
                if (e < total)
                    sz[e] = sv[u] | (((zw[u] >> (4 * (gv[u] & 7))) & 0xFu) << 16);
            }
        }
    }

    // 3. activations of the slice -> LDS (zero past K and in the ring padding),
    //    eight 16-byte loads in flight per thread before any is stored
    {
        const int cpr = nbp * 32;
        const int total = mrows * cpr;
        for (int i0 = 0; i0 < total; i0 += 8 * 64 * T) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = i0 + u * 64 * T + (int)threadIdx.x;
                const int m = min(idx / cpr, mrows - 1), c = min(idx % cpr, nch - 1);
                v[u] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0 + 8 * c);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = i0 + u * 64 * T + (int)threadIdx.x;
                if (idx < total) {
                    const int m = idx / cpr, c = idx % cpr;
                    xs[m * RS + c] = c < nch ? ql::permute_x8(v[u]) : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    }
    __syncthreads();

    // 4. stream the slice: consume block b, refill its slot with block b + P
    f4_t acc[4][MT / 16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < MT / 16; ++t)
            acc[i][t] = f4_t{0.f, 0.f, 0.f, 0.f};
    int arow[MT / 16];
#pragma unroll
    for (int t = 0; t < MT / 16; ++t) {
        const int m = t * 16 + r16;
        arow[t] = (m < mrows ? m : mrows - 1) * RS + 4 * q;
    }
    const uint32_t* szrow = sz + (wave * 16 + r16) * gs;
    const int glane = (32 * q) >> lg;             // this lane's group offset within a block
    const int gmax = gs - 1;

    for (int b0 = 0; b0 < nbp; b0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int b = b0 + p;
            // groups of the two pieces (padding blocks clamp to the last group;
            // their activations are zero)
            const int ga = min(((256 * b) >> lg) + glane, gmax);
            const int gb = min(((256 * b + 128) >> lg) + glane, gmax);
            const uint32_t ea = szrow[ga], eb = szrow[gb];
            const h2_t zb[2] = {ql::zero_bias(ea >> 16), ql::zero_bias(eb >> 16)};
            const h2_t s2[2] = {ql::scale2(ea & 0xFFFFu), ql::scale2(eb & 0xFFFFu)};
            const uint4 w0 = ring[p][0], w1 = ring[p][1];
            const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            h8_t bw[8];
            ql::dequant_block8(words, zb, s2, bw);
            // Refill in place and in order.  Without the scheduling barriers the
            // compiler sinks and regroups the refills, so waiting for one block
            // means waiting for the whole ring.
            const int nxt = b + P < nb ? b + P : nb - 1;
            __builtin_amdgcn_sched_barrier(0);
            load_block(nxt, ring[p][0], ring[p][1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int t = 0; t < MT / 16; ++t) {
                    const int c = b * 32 + (j >> 2) * 16 + (j & 3);
                    const h8_t af = __builtin_bit_cast(h8_t, xs[arow[t] + c]);
                    acc[j & 3][t] = mfma16x16x32(af, bw[j], acc[j & 3][t]);
                }
        }
    }
    f4_t res[MT / 16];
#pragma unroll
    for (int t = 0; t < MT / 16; ++t)
        res[t] = (acc[0][t] + acc[1][t]) + (acc[2][t] + acc[3][t]);

    if (S == 1) {
#pragma unroll
        for (int t = 0; t < MT / 16; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t * 16 + 4 * q + r;
                if (m < M && nok)
                    y[(int64_t)m * N + n] = f32_to_f16_bits(res[t][r]);
            }
        return;
    }

    // 5. split-K: publish this slice's partial tile -- [M][16T] fp32, row-major,
    //    at part[(slice * nblk + column block) * M * 16T] -- with agent-scope
    //    stores, wait for them, then arrive
    constexpr int TW = 16 * T;                    // tile width (columns)
    const int nblk = gridDim.x;
    float* tile = part + ((int64_t)blockIdx.y * nblk + blockIdx.x) * (int64_t)M * TW;
#pragma unroll
    for (int t = 0; t < MT / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = t * 16 + 4 * q + r;
            if (m < M)
                __hip_atomic_store(&tile[m * TW + wave * 16 + r16], res[t][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(0);      // this thread's partial stores have completed
    __syncthreads();                    // ... and so have every other thread's
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&cnt[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!s_last)
        return;
    // The last arrival sums the S tiles in slice order.  Each thread owns four
    // consecutive columns of one row; the slices' 16-byte pieces are read with
    // agent-scope buffer loads, eight slices in flight at a time.
    {
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(part, (uint32_t)((int64_t)S * nblk * M * TW * (int64_t)sizeof(float)));
        constexpr int kSc1 = 16;                  // cache policy: agent scope (bypasses this CU's L1)
        const uint32_t tile_bytes = (uint32_t)(M * TW * sizeof(float));
        const uint32_t col_bytes = (uint32_t)blockIdx.x * tile_bytes;
        const uint32_t slice_bytes = (uint32_t)nblk * tile_bytes;
        for (int v = threadIdx.x; v < M * (TW / 4); v += 64 * T) {
            const uint32_t off = col_bytes + (uint32_t)v * 16u;
            f4_t sum = f4_t{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < S; s0 += 8) {
                f4_t pv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int sl = min(s0 + u, S - 1);
                    pv[u] = __builtin_bit_cast(
                        f4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (int)(off + (uint32_t)sl * slice_bytes), 0,
                                                                    kSc1));
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + u < S)
                        sum += pv[u];
            }
            const int m = v / (TW / 4), nn = n0 + (v % (TW / 4)) * 4;
            uint16_t* yr = y + (int64_t)m * N;
            if (nn + 3 < N && (N & 3) == 0) {
                uint2 h;
                h.x = f32_to_f16_bits(sum[0]) | ((uint32_t)f32_to_f16_bits(sum[1]) << 16);
                h.y = f32_to_f16_bits(sum[2]) | ((uint32_t)f32_to_f16_bits(sum[3]) << 16);
                *reinterpret_cast<uint2*>(yr + nn) = h;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (nn + e < N)
                        yr[nn + e] = f32_to_f16_bits(sum[e]);
            }
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// GEMM (m > 32): block tile BM x BN, K advanced in tiles of 64, 4 waves as
// 2 x 2 (wave tile BM/2 x BN/2), MFMA f32 16x16x32 f16.
//
// Per k-tile the activations (BM rows x 64 k, 128 contiguous bytes per row)
// and the packed weights (BN rows x 8 words) are fetched into registers while
// the previous tile is multiplied.  The weights are dequantised by the shared
// routine as they are written to LDS, once per workgroup, so every wave reads
// both operands as fp16 fragments in the dequantiser's element order.  LDS is
// double-buffered, rows padded to 144 bytes against bank conflicts.  Tiles are
// ordered per XCD as in the int8 GEMM.
// ---------------------------------------------------------------------------
constexpr int kGBK = 64;                  // k per tile
constexpr int kGRow = kGBK * 2 + 16;      // padded LDS row (bytes)
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_tile(int wg, int ntiles)
{
    const int per = (ntiles + kXcds - 1) / kXcds;
    return (wg % kXcds) * per + wg / kXcds;
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void w4a16_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ sc,
                                                         const uint32_t* __restrict__ qz,
                                                         uint16_t* __restrict__ y, int M, int N, int K, int lg)
{
    constexpr int TM = BM / 2, TN = BN / 2;
    constexpr int FI = TM / 16, FJ = TN / 16;
    constexpr int ACH = BM * (kGBK / 8) / 256;         // activation 16-byte chunks per thread per tile
    constexpr int BCH = (BN * 2 + 255) / 256;          // packed 16-byte pieces per thread (2 per row)
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * kGRow];
    uint8_t* const As = lds;
    uint8_t* const Bs = lds + 2 * BM * kGRow;

    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int tile = xcd_tile(blockIdx.x, tm * tn);
    if (tile >= tm * tn)
        return;
    const int m0 = (tile / tn) * BM, n0 = (tile % tn) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, r16 = lane & 15;
    const int KW = K >> 3, NG = K >> lg, ZW = (NG + 7) >> 3;

    uint4 ra[ACH], rb[BCH];
    uint32_t rs[BCH], rz[BCH];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int u = 0; u < ACH; ++u) {
            const int c = tid + u * 256;
            const int row = c >> 3, col = (c & 7) * 8;
            const int m = m0 + row, k = kb + col;
            const bool ok = m < M && k < K;
            ra[u] = *reinterpret_cast<const uint4*>(x + (int64_t)(ok ? m : 0) * K + (ok ? k : 0));
            if (!ok)
                ra[u] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < BCH; ++u) {
            const int c = tid + u * 256;
            const int row = c >> 1, k = kb + (c & 1) * 32;
            const int n = n0 + row;
            const bool ok = row < BN && n < N && k < K;
            const int nn = ok ? n : 0, kk = ok ? k : 0;
            rb[u] = *reinterpret_cast<const uint4*>(qw + (int64_t)nn * KW + (kk >> 3));
            const int g = kk >> lg;
            rs[u] = sc[(int64_t)nn * NG + g];
            rz[u] = qz[(int64_t)nn * ZW + (g >> 3)] >> (4 * (g & 7));
            if (!ok) {
                rb[u] = make_uint4(0u, 0u, 0u, 0u);
                rs[u] = 0u;
                rz[u] = 0u;
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < ACH; ++u) {
            const int c = tid + u * 256;
            *reinterpret_cast<uint4*>(As + buf * BM * kGRow + (c >> 3) * kGRow + (c & 7) * 16) =
                ql::permute_x8(ra[u]);
        }
#pragma unroll
        for (int u = 0; u < BCH; ++u) {
            const int c = tid + u * 256;
            const int row = c >> 1;
            if (row < BN) {
                const h2_t zb = ql::zero_bias(rz[u] & 0xFu), s2 = ql::scale2(rs[u]);
                const uint32_t words[4] = {rb[u].x, rb[u].y, rb[u].z, rb[u].w};
                uint8_t* dst = Bs + buf * BN * kGRow + row * kGRow + (c & 1) * 64;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<h8_t*>(dst + j * 16) = ql::dequant_word8(words[j], zb, s2);
            }
        }
    };

    f4_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + kGBK - 1) / kGBK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            fetch((kt + 1) * kGBK);
        const uint8_t* a_base = As + buf * BM * kGRow + (wm * TM + r16) * kGRow + q * 16;
        const uint8_t* b_base = Bs + buf * BN * kGRow + (wn * TN + r16) * kGRow + q * 16;
#pragma unroll
        for (int s2 = 0; s2 < kGBK / 32; ++s2) {
            h8_t af[FI], bf[FJ];
#pragma unroll
            for (int i = 0; i < FI; ++i)
                af[i] = *reinterpret_cast<const h8_t*>(a_base + i * 16 * kGRow + s2 * 64);
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                bf[j] = *reinterpret_cast<const h8_t*>(b_base + j * 16 * kGRow + s2 * 64);
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
                    acc[i][j] = mfma16x16x32(bf[j], af[i], acc[i][j]);
        }
        if (kt + 1 < nk)
            stash(buf ^ 1);
        __syncthreads();
    }

    // The weight fragment is the MFMA's A operand, so fragment (i, j) is the
    // transposed product: lane (q, r16) holds y[m][n .. n+3], four consecutive
    // outputs of one row.
    const bool vec = m0 + BM <= M && n0 + BN <= N && (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int m = m0 + wm * TM + i * 16 + r16;
            const int n = n0 + wn * TN + j * 16 + 4 * q;
            if (vec) {
                uint2 h;
                h.x = f32_to_f16_bits(acc[i][j][0]) | ((uint32_t)f32_to_f16_bits(acc[i][j][1]) << 16);
                h.y = f32_to_f16_bits(acc[i][j][2]) | ((uint32_t)f32_to_f16_bits(acc[i][j][3]) << 16);
                *reinterpret_cast<uint2*>(y + (int64_t)m * N + n) = h;
            } else if (m < M) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        y[(int64_t)m * N + n + r] = f32_to_f16_bits(acc[i][j][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// GEMM, pipelined (K % 128 == 0): block tile BM x BN, 4 waves, MFMA
// f32 16x16x32 f16 with the weight fragment as the A operand (the accumulator
// is the transposed tile, so each lane ends with four consecutive outputs of
// one row).
//
// K advances in blocks of 128.  Everything a block needs -- activations (BM
// rows x 256 bytes), packed weights (BN rows x 64 bytes), each weight row's
// zero-point word and scales -- is streamed by direct global->LDS loads into
// a ring of S stages, so the main loop issues no other global loads and each
// wave's outstanding-load count is known exactly.  The weights stay packed in
// LDS and are dequantised in registers right before the MFMA by the shared
// routine.
//
// k order inside a block: at MFMA step s (0..3) the lane of quarter q covers
// k = 32q + 8s + [0..7], i.e. word 4q + s of its weight row.  One 16-byte LDS
// read per weight fragment and block gives the lane its words for all four
// steps, and the lane's k range sits in one quantisation group for G = 32, 64
// and 128 alike: one scale and one zero point per fragment and block.  The
// weights are dequantised in natural element order, so the activation chunk
// 4q + s read from LDS is the MFMA operand as it stands.
//
// Waves are laid out WM x WN over the tile.  With 1 x 4 each wave owns BN/4
// weight columns over all BM rows, so every weight word is dequantised by
// exactly one wave and each dequantised fragment feeds BM/16 MFMAs.
//
// Per stage and weight row the ring holds the zero-point word of the block's
// groups and two scale dwords: groups 4kb..4kb+3 (G = 32), 2kb, 2kb+1
// (G = 64, second dword unused), or the aligned pair holding group kb
// (G = 128, second dword unused; this needs an even number of blocks so the
// pair never runs past the end of the scales).
//
// Tiles go to XCDs in groups of GM m-tiles (m fastest within a group), so the
// 32 workgroups an XCD runs at once share a few activation and weight panels.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int S_, int GM_>
struct W4PipeCfg {
    static constexpr int BM = BM_, BN = BN_, S = S_, GM = GM_;
    static constexpr int WM = WM_, WN = 4 / WM_;       // waves along m and n
    static constexpr int kArow = 256;                  // activation LDS row: 128 fp16
    static constexpr int kBrow = 64;                   // weight LDS row: 16 packed words
    static constexpr int kAbytes = BM * kArow, kBbytes = BN * kBrow;
    static constexpr int kZoff = kAbytes + kBbytes;    // zero-point words [BN]
    static constexpr int kSoff = kZoff + BN * 4;       // scale dwords [2][BN]
    static constexpr int kStageBytes = kSoff + BN * 8;
    static constexpr int kLds = S * kStageBytes;
    static constexpr int DA = kAbytes / 4096, DB = kBbytes / 4096;   // 1 KiB loads per wave per stage
    static constexpr int kDwRows = BN / 64;             // 4-byte loads (64 rows each) per table
    static constexpr int DW = (4 * kDwRows + 3) / 4;   // per wave: zero words, scale dwords 0 and 1
    static constexpr int D = DA + DB + DW;
    static_assert(kAbytes % 4096 == 0 && kBbytes % 4096 == 0, "whole 1 KiB loads for every wave");
    static_assert(WM * WN == 4 && BM % (16 * WM) == 0 && BN % (16 * WN) == 0 && BN % 64 == 0,
                  "4 waves of 16-row fragments, 64-row tables");
    static_assert(kStageBytes % 256 == 0, "stages keep the 256-byte row bank alignment");
};

// Scheduling hint for one MFMA step: its LDS reads first, then each MFMA
// followed by up to V vector-ALU instructions (the next step's
// dequantisation), so the matrix pipe and the vector ALU overlap within the
// one wave a SIMD runs.
template <int NDS, int NMFMA, int V>
__device__ __forceinline__ void interleave()
{
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);   // LDS reads
#pragma unroll
    for (int k = 0; k < NMFMA; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // vector ALU
    }
}

// 4-byte direct load: each lane's dword at `src` -> LDS `lds_base` + 4 * lane
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base)
{
    asm volatile("global_load_lds_dword %1, off" : : "{m0}"(lds_base), "v"(src) : "memory");
}

template <class C>
__global__ __launch_bounds__(256) void w4a16_gemm_pipe_kernel(const uint16_t* __restrict__ x,
                                                              const uint32_t* __restrict__ qw,
                                                              const uint16_t* __restrict__ sc,
                                                              const uint32_t* __restrict__ qz,
                                                              uint16_t* __restrict__ y, int M, int N, int K, int lg)
{
    constexpr int BM = C::BM, BN = C::BN, S = C::S, D = C::D, DA = C::DA, DB = C::DB;
    constexpr int TM = BM / C::WM, TN = BN / C::WN;
    constexpr int FI = TM / 16, FJ = TN / 16;
    constexpr int U = S % 2 == 0 ? S : 2 * S;          // unrolled blocks: slot and register parity static
    static_assert(S >= 2 && D * (S - 1) < 64, "ring depth within vmcnt");
    extern __shared__ __attribute__((aligned(1024))) uint8_t pl[];   // S * kStageBytes

    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int tile = xcd_tile(blockIdx.x, tm * tn);
    if (tile >= tm * tn)
        return;
    const int gsz = C::GM * tn;                        // tiles per group of GM m-tiles
    const int grp = tile / gsz, first = grp * C::GM;
    const int gm = min(tm - first, C::GM);
    const int m0 = (first + (tile - grp * gsz) % gm) * BM;
    const int n0 = ((tile - grp * gsz) / gm) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int q = lane >> 4, r16 = lane & 15;
    const uint32_t lds0 = (uint32_t)(uintptr_t)pl;
    const int NG = K >> lg, ZW = (NG + 7) >> 3;
    const int gsh = lg - 4;                            // block kb's first group is kb << (7 - lg)

    // Ring loads of this wave.  Activations: 1 KiB = 4 rows of 256 bytes,
    // lane l writes physical chunk l % 16 of row l / 16.  Weights: 1 KiB =
    // 16 rows of 64 bytes, lane l writes physical chunk l % 4 of row l / 4.
    // Tables: 64 rows of 4 bytes per load; load t (of 4 * BN/64, spread over
    // the waves) is zero words (t / kDwRows == 0), scale dword 0 (1), scale
    // dword 1 (2, G = 32 only, else a repeat of dword 0) or a repeat of the
    // zero words (3).  Rows past M or N re-read the last row (never stored).
    const uint8_t* src[D];
    uint32_t dst[D];
    int step[D];                                       // bytes per block (tables: see issue)
#pragma unroll
    for (int u = 0; u < D; ++u) {
        if (u < DA) {
            const int blk = wave + 4 * u;
            const int row = blk * 4 + (lane >> 4);
            const int c = (lane & 15) ^ ql::swz256(row);
            const int m = min(m0 + row, M - 1);
            src[u] = reinterpret_cast<const uint8_t*>(x) + (int64_t)m * K * 2 + 16 * c;
            dst[u] = (uint32_t)(blk * 1024);
            step[u] = 256;
        } else if (u < DA + DB) {
            const int blk = wave + 4 * (u - DA);
            const int row = blk * 16 + (lane >> 2);
            const int c = (lane & 3) ^ ql::swz64(row);
            const int n = min(n0 + row, N - 1);
            src[u] = reinterpret_cast<const uint8_t*>(qw) + (int64_t)n * (K / 2) + 16 * c;
            dst[u] = (uint32_t)(C::kAbytes + blk * 1024);
            step[u] = 64;
        } else {
            const int t = wave + 4 * (u - DA - DB);
            const int kind = t / C::kDwRows, part = t % C::kDwRows;
            const int row = 64 * part + lane;
            const int n = min(n0 + row, N - 1);
            if (kind == 1 || kind == 2) {
                const int extra = (kind == 2 && lg == 5) ? 4 : 0;
                src[u] = reinterpret_cast<const uint8_t*>(sc) + (int64_t)n * NG * 2 + extra;
                dst[u] = (uint32_t)(C::kSoff + (kind == 2 ? 4 * BN : 0) + 4 * 64 * part);
                step[u] = -1;                          // scale dwords
            } else {
                src[u] = reinterpret_cast<const uint8_t*>(qz) + (int64_t)n * ZW * 4;
                dst[u] = (uint32_t)(C::kZoff + 4 * 64 * part);
                step[u] = -2;                          // zero words
            }
        }
    }
    auto issue = [&](int kb, int slot) {
        const uint32_t sbase = lds0 + slot * C::kStageBytes;
        // scale byte offset of block kb: first group * 2, aligned down to 4
        const int soff = ((kb << (7 - lg)) * 2) & ~3;
        const int zoff = 4 * (kb >> gsh);
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (u < DA + DB) {
                ql::dma16(src[u] + (int64_t)kb * step[u], (uint32_t)__builtin_amdgcn_readfirstlane(sbase + dst[u]));
            } else {
                // 64 rows x 4 bytes, lane l -> row 64 * part + l
                const bool is_scale = step[u] == -1;
                const uint8_t* p = src[u] + (is_scale ? soff : zoff);
                dma4(p, (uint32_t)__builtin_amdgcn_readfirstlane(sbase + dst[u]));
            }
        }
    };


    // LDS fragment reads: activations of step st (FI fragments), the packed
    // weight words of a block (FJ fragments), and the block's zero-point word
    // and scale for each weight fragment
    auto read_a = [&](int slot, int st, uint4 (&fa)[FI]) {
        const uint8_t* base = pl + slot * C::kStageBytes;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int r = wm * TM + 16 * i + r16;
            fa[i] = *reinterpret_cast<const uint4*>(base + r * C::kArow + 16 * ((4 * q + st) ^ ql::swz256(r)));
        }
    };
    auto read_b = [&](int slot, int kb, uint4 (&fb)[FJ], uint32_t (&zr)[FJ], uint32_t (&sr)[FJ]) {
        const uint8_t* base = pl + slot * C::kStageBytes;
        // scale of this lane's group: table and half within the dword
        const int tbl = lg == 5 ? (q >> 1) : 0;
        const int half = lg == 7 ? (kb & 1) : (lg == 6 ? (q >> 1) : (q & 1));
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int r = wn * TN + 16 * j + r16;
            fb[j] = *reinterpret_cast<const uint4*>(base + C::kAbytes + r * C::kBrow + 16 * (q ^ ql::swz64(r)));
            zr[j] = *reinterpret_cast<const uint32_t*>(base + C::kZoff + 4 * r);
            sr[j] = *reinterpret_cast<const uint16_t*>(base + C::kSoff + tbl * 4 * BN + 4 * r + 2 * half);
        }
    };

    f4_t acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    uint4 fa[2][FI], fb[2][FJ];
    uint32_t zr[2][FJ], sr[2][FJ];
    h2_t zb[2][FJ], s2[2][FJ];
    h8_t bw[2][FJ];
    const int nk = K / 128;
    auto word = [](const uint4& w4, int st) { return st == 0 ? w4.x : st == 1 ? w4.y : st == 2 ? w4.z : w4.w; };
    // zero bias and scale of block kb from its table words
    auto set_zs = [&](int kb, int p) {
        const int zsh = 4 * (((kb * 128 + 32 * q) >> lg) & 7);
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            zb[p][j] = ql::zero_bias((zr[p][j] >> zsh) & 0xFu);
            s2[p][j] = ql::scale2(sr[p][j]);
        }
    };
    auto dequant = [&](int p, int st, h8_t (&out)[FJ]) {
        uint32_t w[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            w[j] = word(fb[p][j], st);
        ql::dequant_words_natural<FJ>(w, zb[p], s2[p], out);
    };
    auto mfmas = [&](int cur, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = mfma16x16x32(bw[cur][j], __builtin_bit_cast(h8_t, fa[cur][i]), acc[i][j]);
    };

#pragma unroll
    for (int s = 0; s < S; ++s)
        issue(s < nk ? s : nk - 1, s);
    ql::stage_barrier<D * (S - 1)>();   // block 0 landed
    read_a(0, 0, fa[0]);
    read_b(0, 0, fb[0], zr[0], sr[0]);
    set_zs(0, 0);
    dequant(0, 0, bw[0]);

    // One block.  fa[st & 1] / bw[st & 1] hold step st's operands, prepared
    // during step st-1.  Step 3 waits for the next block (S-2 younger blocks
    // may still be in flight), refills this block's slot and reads the next
    // block's weights, tables and first activation fragments, whose
    // dequantisation fills the second half of step 3.  Every load is issued
    // unconditionally (block indices clamped to the last block), so every wave
    // has exactly D * (S-2) loads younger than the block it waits for.
    auto block = [&](int kb, int u) {
        const int slot = u % S, par = u & 1;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int cur = st & 1;
            if (st < 3) {
                read_a(slot, st + 1, fa[cur ^ 1]);
                dequant(par, st + 1, bw[cur ^ 1]);
                mfmas(cur, 0, FI);
                interleave<FI, FI * FJ, 3>();
            } else {
                ql::stage_barrier<D * (S - 2)>();
                issue(min(kb + S, nk - 1), slot);
                read_b((u + 1) % S, kb + 1, fb[par ^ 1], zr[par ^ 1], sr[par ^ 1]);
                read_a((u + 1) % S, 0, fa[cur ^ 1]);
                mfmas(cur, 0, FI / 2);
                set_zs(kb + 1, par ^ 1);
                dequant(par ^ 1, 0, bw[cur ^ 1]);
                mfmas(cur, FI / 2, FI);
                interleave<FI + 3 * FJ, FI * FJ, 3>();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int kb0 = 0;
    for (; kb0 + U <= nk; kb0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            block(kb0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb0 + u < nk)
            block(kb0 + u, u);
    ql::stage_barrier<0>();   // drain the trailing reloads before the workgroup exits

    // lane (q, r16) holds y[m][n .. n+3] of fragment (i, j)
    const bool vec = m0 + BM <= M && n0 + BN <= N && (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int m = m0 + wm * TM + i * 16 + r16;
            const int n = n0 + wn * TN + j * 16 + 4 * q;
            if (vec) {
                uint2 h;
                h.x = f32_to_f16_bits(acc[i][j][0]) | ((uint32_t)f32_to_f16_bits(acc[i][j][1]) << 16);
                h.y = f32_to_f16_bits(acc[i][j][2]) | ((uint32_t)f32_to_f16_bits(acc[i][j][3]) << 16);
                *reinterpret_cast<uint2*>(y + (int64_t)m * N + n) = h;
            } else if (m < M) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        y[(int64_t)m * N + n + r] = f32_to_f16_bits(acc[i][j][r]);
            }
        }
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct DecodePlan {
    int mt;     // 16 or 32
    int t;      // waves (16-channel tiles) per workgroup
    int p;      // blocks in flight per wave
    int ks;     // k per slice (multiple of 256)
    int slices; // split-K factor
    int nblk;   // column blocks
    size_t lds_bytes;   // dynamic LDS bytes
    size_t part_offset, part_bytes;
};

// The workspace starts with a fixed counter region that only ever holds
// arrival counters (zero between calls); partial sums follow it.  A fixed
// region keeps calls of different shapes from reading each other's partial
// sums as counters when they share one workspace.
constexpr size_t kCounterBytes = 32768;
constexpr int kMaxDecodeBlocks = (int)(kCounterBytes / sizeof(uint32_t));
constexpr size_t kDecodeLdsBudget = 80 * 1024;   // staged activations + scales per workgroup (two per CU)
constexpr int kDecodeWaveTarget = 2048;          // >= 8 streaming waves per CU

// Tile choice.  Activations of one slice are staged per workgroup, so the
// slice length is capped by the LDS budget (two workgroups per CU); within that cap the slice is
// as long as possible (fewer partial sums), but K is split further when the
// column tiles alone give fewer than ~8 streaming waves per CU.
DecodePlan decode_plan(int64_t m, int64_t n, int64_t k, int group)
{
    DecodePlan p{};
    p.mt = m <= 16 ? 16 : 32;
    p.t = 4;
    p.nblk = (int)((n + p.t * 16 - 1) / (p.t * 16));
    const int64_t rows = std::min<int64_t>(m, p.mt);
    const int64_t kblocks = (k + 255) / 256;
    const int64_t waves = (int64_t)p.nblk * p.t;
    int64_t slices = waves >= kDecodeWaveTarget ? 1 : (kDecodeWaveTarget + waves - 1) / waves;
    slices = std::min<int64_t>(slices, kblocks);
    for (;; ++slices) {
        const int64_t sblocks = (kblocks + slices - 1) / slices;
        const int pd = 2;   // a ring of 2 measured at least as fast as 4 on every MLP decode shape
        const int64_t nbp = (sblocks + pd - 1) / pd * pd;
        const int64_t gs = sblocks * 256 / group;
        const size_t lds = (size_t)rows * (size_t)(nbp * 32 + 1) * 16 + (size_t)(16 * p.t * gs) * 4;
        if (lds <= kDecodeLdsBudget || sblocks == 1) {
            p.p = pd;
            p.ks = (int)(sblocks * 256);
            p.lds_bytes = lds;
            break;
        }
    }
    p.slices = (int)((k + p.ks - 1) / p.ks);
    p.part_offset = kCounterBytes;
    // partial tiles [slices][nblk][m][16 t] fp32
    p.part_bytes = p.slices > 1 ? (size_t)p.slices * (size_t)p.nblk * (size_t)m * (size_t)(16 * p.t) * sizeof(float)
                                : 0;
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
    if (n > (1LL << 30) || k > (1LL << 30) || n * (k / 2) >= (1LL << 31))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: n=%lld k=%lld: packed weights must stay below 2 GiB", who, (long long)n,
                (long long)k);
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

template <int MT, int T, int P>
void launch_decode_t(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                     const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int lg, hipStream_t st)
{
    uint32_t* cnt = p.slices > 1 ? static_cast<uint32_t*>(ws) : nullptr;
    float* part = p.slices > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_offset) : nullptr;
    hipLaunchKernelGGL((w4a16_decode_kernel<MT, T, P>), dim3(p.nblk, p.slices), dim3(64 * T), p.lds_bytes, st, x, qw,
                       sc, qz, y, part, cnt, m, n, k, lg, p.ks);
}

// Exact dispatch on the plan; returns false for a combination that is not
// instantiated.
bool launch_decode(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                   const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int lg, hipStream_t st)
{
#define QL_DECODE_CASE(MT_, T_, P_)                                                    \
    if (p.mt == MT_ && p.t == T_ && p.p == P_) {                                       \
        launch_decode_t<MT_, T_, P_>(p, x, qw, sc, qz, y, ws, m, n, k, lg, st);        \
        return true;                                                                   \
    }
    QL_DECODE_CASE(16, 4, 2) QL_DECODE_CASE(32, 4, 2)
#undef QL_DECODE_CASE
    return false;
}

}  // namespace

extern "C" size_t ql_w4a16_workspace_bytes(int64_t m, int64_t n, int64_t k, int group)
{
    (void)group;
    if (m <= 0 || n <= 0 || k <= 0 || m > 32)
        return 0;
    return decode_workspace(decode_plan(m, n, k, group));
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
        DecodePlan p = decode_plan(m, n, k, group);
        if (p.slices > 1 && p.nblk > kMaxDecodeBlocks)
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: n=%lld exceeds the decode path's %d column blocks", who, (long long)n,
                    kMaxDecodeBlocks);
        if (p.part_bytes >= ((size_t)1 << 32))
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: m=%lld n=%lld k=%lld needs %zu bytes of partial sums (limit 4 GiB)", who,
                    (long long)m, (long long)n, (long long)k, p.part_bytes);
        const size_t need = decode_workspace(p);
        if (need > 0 && (!workspace || workspace_bytes < need))
            QL_FAIL(QL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    workspace ? workspace_bytes : (size_t)0);
        if (need > 0 && !ql::aligned16(workspace))
            QL_FAIL(QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
        const int lg = group == 32 ? 5 : (group == 64 ? 6 : 7);
        if (!launch_decode(p, xw, qw, scales, qz, y, workspace, mi, ni, ki, lg, st))
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: no decode kernel for mt=%d t=%d p=%d", who, p.mt, p.t, p.p);
        return launch_status(who);
    }
    const int lg = group == 32 ? 5 : (group == 64 ? 6 : 7);
    // 128 x 192 tiles: M=512, N=12288 gives exactly one tile per CU
    constexpr int BM = 128, BN = 192;
    using Pipe = W4PipeCfg<BM, BN, 1, 3, 4>;
    const int64_t tiles = ((n + BN - 1) / BN) * ((m + BM - 1) / BM);
    const unsigned grid = (unsigned)((tiles + kXcds - 1) / kXcds * kXcds);   // whole rounds over the XCDs
    // G = 128 reads scale pairs, which needs an even number of 128-blocks
    if (k % 128 == 0 && (group != 128 || (k / 128) % 2 == 0) && ql::lds_fits(Pipe::kLds))
        hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe>), dim3(grid), dim3(256), (size_t)Pipe::kLds, st, xw, qw,
                           scales, qz, y, mi, ni, ki, lg);
    else
        hipLaunchKernelGGL((w4a16_gemm_kernel<BM, BN>), dim3(grid), dim3(256), 0, st, xw, qw, scales, qz, y, mi, ni,
                           ki, lg);
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
