// W4A16 kernels for gfx950 and their C-ABI entry points.
//
//   w4a16_dequant_kernel  -- writes the shared dequantisation routine's output
//   w4a16_decode_kernel   -- 4 <= m <= 64: split-K GEMV on MFMA, weights
//                            streamed from HBM once, dequantised in registers
//   w4a16_gemv_kernel     -- m <= 3: one 16-channel tile per workgroup, K split
//                            among its waves, activations and tables in LDS
//   w4a16_gemm_pipe_kernel -- m > 64: LDS-ring fp16 MFMA GEMM (split-K when
//                            its tiles would leave CUs idle)
//   w4a16_gemm_kernel     -- the same for shapes the ring does not cover
//
// Weight format (LMDeploy walkthrough, section 2; AUQ page, section 5.4):
// qweight int32 [n, k/8] with code i of a word at bits [4i, 4i+4), fp16 scales
// [n, k/group], uint4 zero points packed eight to an int32 [n, ceil(k/group/8)].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

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
// dequant export: one thread per 8-word block of a row (the row length K/8 is
// a multiple of 8 words when K is a multiple of 64; otherwise the last block
// of a row is partial).  Even blocks take the interleaved routine (put back
// in natural order), odd blocks the natural one, so the exported weights check
// both.  Words 0-3 and 4-7 of a block each lie in one group (G >= 32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4a16_dequant_kernel(const uint32_t* __restrict__ qw,
                                                            const uint16_t* __restrict__ sc,
                                                            const uint32_t* __restrict__ qz,
                                                            uint16_t* __restrict__ w16,
                                                            uint8_t* __restrict__ q8, int N, int K, int G)
{
    const int KW = K / 8, NG = K / G, ZW = (NG + 7) / 8;
    const int BPR = (KW + 7) / 8;                     // blocks per row
    const int64_t total = (int64_t)N * BPR;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int n = (int)(i / BPR), jb = (int)(i - (int64_t)n * BPR);
        const int j0 = jb * 8, nw = min(8, KW - j0);
        uint32_t w[8];
        ql::zb_t zb[8];
        h2_t s2[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + min(u, nw - 1);
            const int g = (8 * j) / G;
            w[u] = qw[(int64_t)n * KW + j];
            zb[u] = ql::make_zb(ql::zero_of(qz + (int64_t)n * ZW, g));
            s2[u] = ql::scale2(sc[(int64_t)n * NG + g]);
        }
        h8_t v[8];
        if ((jb & 1) == 0) {
            ql::dequant_words<8>(w, zb, s2, v);
        } else {
            ql::dequant_words_natural<8>(w, zb, s2, v);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u >= nw)
                break;
            uint4 o = __builtin_bit_cast(uint4, v[u]);
            if ((jb & 1) == 0) {
                const uint32_t a = o.x, b = o.y, c = o.z, d = o.w;   // (0,4)(1,5)(2,6)(3,7)
                o.x = (a & 0xFFFFu) | (b << 16);
                o.y = (c & 0xFFFFu) | (d << 16);
                o.z = (a >> 16) | (b & 0xFFFF0000u);
                o.w = (c >> 16) | (d & 0xFFFF0000u);
            }
            const int64_t wi = (int64_t)n * KW + j0 + u;
            *reinterpret_cast<uint4*>(w16 + wi * 8) = o;
            if (q8) {
                const uint32_t ww = w[u];
                uint2 cq;
                cq.x = (ww & 0xFu) | ((ww >> 4) & 0xFu) << 8 | ((ww >> 8) & 0xFu) << 16 | ((ww >> 12) & 0xFu) << 24;
                cq.y = ((ww >> 16) & 0xFu) | ((ww >> 20) & 0xFu) << 8 | ((ww >> 24) & 0xFu) << 16 | (ww >> 28) << 24;
                *reinterpret_cast<uint2*>(q8 + wi * 8) = cq;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// decode: m <= MT (16, 32 or 64)
//
// Workgroup = T waves (4, or 6 where that keeps every CU at one workgroup; 8
// for 64 rows, one workgroup per CU);
// wave w owns R tiles of 16 output channels, so a workgroup covers
// TW = 16 T R channels and one K slice of KS (a multiple of 256; one slice
// when K is not split).  K advances in blocks of 256.  Per
// block each wave streams its rows' weights through a P-deep register ring,
// and the workgroup streams the block's activations (rows < m) through a
// two-slot LDS ring: the threads load block b + P's activations together with
// the weights of block b + P, reorder each 16-byte chunk for the dequantiser
// in registers and write it to LDS one block ahead of its use; one barrier per
// block publishes it.  With XB = 2 (the six-wave 16-row launches, one
// workgroup per CU) the activations are requested four blocks ahead and
// published two at a time into a four-slot ring, one barrier per two blocks.
// Every load is an ordinary (compiler-tracked) load, so each wait names
// exactly the block it needs.
//
// In a block, lane l (row l%16, quarter q = l/16) loads two 16-byte pieces of
// its row: words [4q, 4q+4) and [16+4q, 16+4q+4), so 4 lanes read 64
// contiguous bytes of a row per load.  Word j of piece h is the B operand of
// one MFMA directly; weights never pass through LDS.  An activation fragment
// read from LDS serves all R tiles of the wave.
//
// With 128-channel groups (POST) every MFMA sums 32 k of one group per output
// channel, so the kernel feeds the exact integers q - z and applies the group
// scale to the fp32 result of each group's MFMAs; otherwise the dequantised
// fp16 weights (q - z) * s are fed.
//
// Weights, scales and zero points are read with buffer loads: a scalar
// resource per tensor and a 32-bit per-lane offset.  A read past a resource's
// end returns zero.  Lanes past N read row N-1 and their outputs are
// discarded; pieces past the slice end read finite words of the same tensor
// that meet zero activations.  Activation rows past m are zero in LDS.
//
// Split-K (S > 1 slices): each slice writes its fp32 partial tile with
// agent-scope stores, waits for them to complete, then bumps a per-column-block
// arrival counter; the last arrival reads the partials back with agent-scope
// loads and sums them in slice order (deterministic).  No cache-wide fence is
// needed because every cross-workgroup value travels through agent-scope
// accesses.  With exactly two slices the partials meet in exchange slots
// instead (pair_finish below: one atomic round trip instead of three).
// ---------------------------------------------------------------------------
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcFlags);
}

// Activation blocks in LDS: chunk c (16 bytes) of row m sits at chunk
// c ^ xswz(m) of the row.  The image of xswz never sets bit 2, so for the
// chunks a fragment read touches (16 h + 4q + j, j < 4) the 32 lanes with
// q < 2 -- and the 32 with q >= 2 -- land on 32 distinct chunks of one
// 512-byte span.
__device__ __forceinline__ int xswz(int m) { return (m & 3) | ((m & 12) << 1); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t s16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)s16);
}

// Workgroups per CU the register budget is held to: three four-wave
// workgroups for one 16-row tile (a 1376-wave launch stays resident in one
// round), two for 32 or 64 rows; as many T-wave workgroups as fit the same
// waves (one eight-wave workgroup for 64 rows).  A launch that publishes
// activations every second block (XB = 2: the six-wave, one-workgroup-per-CU
// plans) is held to one workgroup per CU.
template <int MT, int R, int T = 4, int XB = 1>
constexpr int decode_wg_per_cu()
{
    constexpr int waves = 4 * (R > 1 ? 1 : (MT == 16 ? 3 : 2));
    return XB > 1 ? 1 : (waves / T > 0 ? waves / T : 1);
}

// Scale and zero-point tables of TW channels [n0, n0 + TW) for the groups
// [g0, g0 + gs) of a slice, staged in LDS as dwords: per channel SD dwords of
// scales starting at the even element at or below its first group (the dword
// holding it), then per channel ZD words of zero points.  (The scales are read
// in 4-byte units, up to the 4-byte boundary at or after their end.)  load()
// requests a batch of SB scale dwords and ZB zero words per thread (NT
// threads); store_all()
// writes it to LDS, then loads and writes any further batches.  Threads past
// the end rewrite the last entry with its own value, so no load has a
// conditional use the compiler could sink it into; each table has its own loop,
// since a per-lane choice of buffer resource would make the compiler loop over
// the distinct resources.
template <int TW, int SB, int ZB, int NT = 256>
struct DecodeTables {
    __amdgpu_buffer_rsrc_t rsc, rzr;
    int n0, N, NG, ZW, g0, SD, ZD, stot, ztot;
    uint32_t sv[SB], zv[ZB];

    __device__ __forceinline__ DecodeTables(const uint16_t* sc, const uint32_t* qz, int n0_, int N_, int NG_,
                                            int ZW_, int g0_, int gs)
        : n0(n0_), N(N_), NG(NG_), ZW(ZW_), g0(g0_)
    {
        rsc = make_rsrc(sc, ((uint32_t)N * (uint32_t)NG * 2u + 3u) & ~3u);
        rzr = make_rsrc(qz, (uint32_t)N * (uint32_t)ZW * 4u);
        SD = (gs >> 1) + 1;
        ZD = (gs >> 3) + 2;
        stot = TW * SD;
        ztot = TW * ZD;
    }
    __device__ __forceinline__ void load(int e0, int z0)
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int e = min(e0 + u * NT + tid, stot - 1);
            const int rr = e / SD, col = e - rr * SD;
            const uint32_t row = (uint32_t)min(n0 + rr, N - 1);
            const uint32_t dw = ((row * (uint32_t)NG + (uint32_t)g0) >> 1) + (uint32_t)col;
            sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rsc, (int)(dw * 4u), 0, 0);
        }
#pragma unroll
        for (int u = 0; u < ZB; ++u) {
            const int e = min(z0 + u * NT + tid, ztot - 1);
            const int rr = e / ZD, col = e - rr * ZD;
            const uint32_t row = (uint32_t)min(n0 + rr, N - 1);
            const uint32_t wd = row * (uint32_t)ZW + (uint32_t)(g0 >> 3) + (uint32_t)col;
            zv[u] = __builtin_amdgcn_raw_buffer_load_b32(rzr, (int)(wd * 4u), 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint32_t* tab, int e0, int z0) const
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < SB; ++u)
            tab[min(e0 + u * NT + tid, stot - 1)] = sv[u];
#pragma unroll
        for (int u = 0; u < ZB; ++u)
            tab[stot + min(z0 + u * NT + tid, ztot - 1)] = zv[u];
    }
    // the first batch was requested by load(0, 0)
    __device__ __forceinline__ void store_all(uint32_t* tab)
    {
        store(tab, 0, 0);
        for (int e0 = SB * NT, z0 = ZB * NT; e0 < stot || z0 < ztot; e0 += SB * NT, z0 += ZB * NT) {
            load(e0, z0);
            store(tab, e0, z0);
        }
    }
    // element offset of a channel's first group within its scale dwords
    __device__ __forceinline__ int parity(int rr) const
    {
        return (int)(((uint32_t)min(n0 + rr, N - 1) * (uint32_t)NG + (uint32_t)g0) & 1u);
    }
};

// Split-K completion, after this thread's agent-scope stores of its part of
// the workgroup's partial tile ([M][TW] fp32 at part[(slice * nblk + column
// block) * M * TW]): wait for them, arrive on the column block's counter, and
// if this workgroup arrived last, sum the S tiles in slice order and store y.
// Each thread of the last workgroup owns four consecutive columns of one row;
// the slices' 16-byte pieces are read with agent-scope buffer loads, eight
// slices in flight at a time.  The last arrival resets the counter.
template <int TW>
__device__ __forceinline__ void splitk_finish(float* __restrict__ part, uint32_t* __restrict__ cnt,
                                              uint16_t* __restrict__ y, int M, int N, int n0, int* s_last)
{
    const int S = gridDim.y, nblk = gridDim.x, tid = threadIdx.x;
    __builtin_amdgcn_s_waitcnt(0);      // this thread's partial stores have completed
    __syncthreads();                    // ... and so have every other thread's
    if (tid == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&cnt[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (prev == (uint32_t)(S - 1));
    }
    __syncthreads();
    if (!*s_last)
        return;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, (uint32_t)((int64_t)S * nblk * M * TW * (int64_t)sizeof(float)));
    constexpr int kSc1 = 16;                  // cache policy: agent scope (bypasses this CU's L1)
    const uint32_t tile_bytes = (uint32_t)(M * TW * sizeof(float));
    const uint32_t col_bytes = (uint32_t)blockIdx.x * tile_bytes;
    const uint32_t slice_bytes = (uint32_t)nblk * tile_bytes;
    for (int v = tid; v < M * (TW / 4); v += blockDim.x) {
        const uint32_t off = col_bytes + (uint32_t)v * 16u;
        f4_t sum = f4_t{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += 8) {
            f4_t pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sl = min(s0 + u, S - 1);
                pv[u] = __builtin_bit_cast(
                    f4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (int)(off + (uint32_t)sl * slice_bytes), 0, kSc1));
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
    if (tid == 0)
        __hip_atomic_store(&cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two-slice completion.  With K split in exactly two slices every output is
// the sum of two partials, one per slice, added in slice order (slice 0's
// first, which fixes the bits even for NaN payloads).  Each pair of adjacent
// output rows of a lane meets in one 8-byte slot of a region that is zero
// between calls: each slice swaps its two partials into the slot with one
// relaxed agent-scope atomic exchange (the values travel in the atomic
// itself, so nothing else needs ordering, and there is no arrival counter,
// no wait for store acknowledgements and no re-read of partial tiles).  The
// exchange that returns zero came first and is done; the other receives the
// first slice's partials, adds them to its own, stores the fp16 outputs and
// puts zero back.  Slots hold the partials' bits XOR kPairKey, so a zero
// slot cannot be mistaken for stored partials: that would need both partials
// to be 0x7F8A5A5A, a signalling NaN with nonzero low 13 mantissa bits,
// which neither fp32 arithmetic (its NaNs are quiet) nor a value widened
// from fp16 (low 13 bits zero) produces.
//
// NF fragments per lane: fragment f holds output rows row0[f] + 0..3 of
// column col[f]; its slots are slot[(f * 2 + h) * 64 + lane], h = 0 for rows
// 0-1 and 1 for rows 2-3, so each exchange instruction covers 512 contiguous
// bytes (interleaving h, 0.1-0.3 us slower).  Pairs starting at or past M (the padding of the
// row tiles) are skipped by both slices alike: the exchanges' cost grows with
// their number (exchanging the padding too made gate/up M = 4 / 8 0.4 us
// slower).
constexpr uint64_t kPairKey = 0x7F8A5A5A7F8A5A5Aull;

template <int NF>
__device__ __forceinline__ void pair_finish(uint64_t* __restrict__ slot, const f4_t (&v)[NF], const int (&row0)[NF],
                                            const int (&col)[NF], uint16_t* __restrict__ y, int M, int N)
{
    const int lane = threadIdx.x & 63;
    const bool first_slice = blockIdx.y == 0;
    // every exchange's address and operand in registers of its own before
    // the first is issued (computed inside each lane-predicated exchange,
    // they shared registers, and each exchange waited for the one before)
    typedef __attribute__((address_space(1))) uint64_t gu64_t;   // global memory: global, not flat, atomics
    gu64_t* addr[NF][2];
    uint64_t val[NF][2], old[NF][2];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // (each element copied out first: a bit cast of a vector element
            // in place reads element 0)
            const float lo = v[f][2 * h], hi = v[f][2 * h + 1];
            val[f][h] = ((uint64_t)__builtin_bit_cast(uint32_t, lo) |
                         ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32)) ^ kPairKey;
            addr[f][h] = (gu64_t*)&slot[(f * 2 + h) * 64 + lane];
            asm volatile("" : "+v"(val[f][h]), "+v"(addr[f][h]));
        }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            old[f][h] = row0[f] + 2 * h < M ? __hip_atomic_exchange(addr[f][h], val[f][h], __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT)
                                            : 0ull;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (old[f][h] == 0ull)
                continue;
            const uint64_t o = old[f][h] ^ kPairKey;
            const float other[2] = {__builtin_bit_cast(float, (uint32_t)o), __builtin_bit_cast(float, (uint32_t)(o >> 32))};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float mine = v[f][2 * h + e];
                const float sum = first_slice ? mine + other[e] : other[e] + mine;
                const int m = row0[f] + 2 * h + e;
                if (m < M && col[f] < N)
                    y[(int64_t)m * N + col[f]] = f32_to_f16_bits(sum);
            }
            __hip_atomic_store(&slot[(f * 2 + h) * 64 + lane], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
}

// The same exchange for one output per thread: a 4-byte slot holding the
// partial's bits XOR the low half of kPairKey.
__device__ __forceinline__ void pair_finish_one(uint32_t* __restrict__ slot, float v, uint16_t* __restrict__ y, int m,
                                                int col, int N)
{
    constexpr uint32_t kKey = (uint32_t)kPairKey;
    const uint32_t old = __hip_atomic_exchange(slot, __builtin_bit_cast(uint32_t, v) ^ kKey, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    if (old == 0u)
        return;
    const float other = __builtin_bit_cast(float, old ^ kKey);
    const float sum = blockIdx.y == 0 ? v + other : other + v;
    if (col < N)
        y[(int64_t)m * N + col] = f32_to_f16_bits(sum);
    __hip_atomic_store(slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int R, int P, bool POST, int T = 4, int XB = 1>
__global__ __launch_bounds__(64 * T, (decode_wg_per_cu<MT, R, T, XB>())) void w4a16_decode_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int M, int N, int K, int lg, int KS, int pair)
{
    constexpr int NT = 64 * T;                     // threads
    constexpr int TW = 16 * T * R;                 // channels per workgroup
    constexpr int MTI = MT / 16;                   // MFMA row tiles
    constexpr int XC = MT * 32;                    // activation chunks per block
    constexpr int XPT = (XC + NT - 1) / NT;        // ... per thread
    constexpr int NJ = POST ? 1 : (R * MTI >= 4 ? 1 : 4 / (R * MTI));   // accumulator chains
    constexpr int NW = 8 * R;                      // words per lane and block
    // activations: published every XB blocks, so XR blocks are held in
    // registers (requested XR blocks ahead) and XSL in the LDS ring; the loop
    // is unrolled over U blocks (a multiple of both rings)
    static_assert(XB == 1 || (XB == 2 && P == 2), "barrier every block, or every second with a 2-deep ring");
    constexpr int XR = XB == 1 ? P : 4;
    constexpr int XSL = XB == 1 ? 2 : 4;
    constexpr int U = XB == 1 ? P : 4;
    __shared__ uint4 xs[XSL][MT * 32];             // activation ring: XSL 256-k blocks
    extern __shared__ uint32_t tab[];              // scale and zero-point tables
    __shared__ int s_last;

    // K slice: blocks [y nkb / S, (y + 1) nkb / S) of the nkb 256-k blocks,
    // so slices differ by at most one block (KS is the longest)
    const int S = gridDim.y;
    const int nkb = (K + 255) >> 8;
    const int k0 = (int)(((int64_t)blockIdx.y * nkb) / S) << 8;
    const int kend = min(K, (int)(((int64_t)(blockIdx.y + 1) * nkb) / S) << 8);
    const int nch = (kend - k0) >> 3;             // valid chunks of the slice
    const int nb = (kend - k0 + 255) >> 8;        // blocks of this slice
    const int nbp = (nb + U - 1) / U * U;         // blocks streamed, padded to the unrolled step
    const int mrows = M < MT ? M : MT;
    const int gs = KS >> lg;                      // groups per slice

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * TW;
    const int KW = K >> 3, NG = K >> lg, ZW = (NG + 7) >> 3;

    // activation chunks of this thread: chunk tid + NT u of a block is chunk
    // (tid + NT u) % 32 of row (tid + NT u) / 32; with NT not dividing the
    // block's chunks, a thread's last chunk may not exist (xhas)
    int xsrc[XPT], xdst[XPT], xcc[XPT];
    bool xok[XPT], xhas[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int craw = tid + NT * u;
        xhas[u] = craw < XC;
        const int c = xhas[u] ? craw : XC - 1, m = c >> 5, cc = c & 31;
        xok[u] = m < mrows;
        xcc[u] = cc;
        xsrc[u] = (m < mrows ? m : mrows - 1) * K + k0;   // element offset of the row's slice
        xdst[u] = m * 32 + (cc ^ xswz(m));
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    auto x_load = [&](int j, uint4 (&v)[XPT]) {
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const uint32_t e = (uint32_t)(xsrc[u] + 8 * min(j * 32 + xcc[u], nch - 1));
            v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(e * 2u), 0, 0));
        }
    };
    // rows past m and chunks past the slice's end are stored as zeros (the
    // permute's zero selectors), without a branch
    int xlim[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u)
        xlim[u] = xok[u] ? nch : 0;
    auto x_store = [&](int j, const uint4 (&v)[XPT]) {
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const bool ok = j * 32 + xcc[u] < xlim[u];
            if (XC % NT == 0 || xhas[u])
                xs[j % XSL][xdst[u]] =
                    ql::permute_x8_sel(v[u], ok ? ql::kPermLo : ql::kPermZero, ok ? ql::kPermHi : ql::kPermZero);
        }
    };

    // scale and zero-point tables of this workgroup's channels and slice
    const int g0 = k0 >> lg;
    DecodeTables<TW, 6 * R, 2 * R, NT> tb(sc, qz, n0, N, NG, ZW, g0, gs);

    // weights: block b of this lane's tile t, two 16-byte pieces
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)KW * 4u);
    uint32_t ow[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int n = n0 + (wave * R + t) * 16 + r16;
        ow[t] = (uint32_t)(n < N ? n : N - 1) * (uint32_t)KW * 4u + (uint32_t)(k0 + 32 * q) / 2u;
    }
    auto load_block = [&](int b, uint4 (&rg)[R][2]) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const uint32_t bw = ow[t] + (uint32_t)b * 128u;
            rg[t][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)bw, 0, 0));
            rg[t][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(bw + 64u), 0, 0));
        }
    };

    // 1. requests: tables, then activations and weights of the first P blocks
    //    (weights past the slice re-read block nb-1, so every wait in the
    //    stream has a static count)
    tb.load(0, 0);
    uint4 ring[P][R][2];
    uint4 xr[XR][XPT];
#pragma unroll
    for (int p = 0; p < (XR > P ? XR : P); ++p) {
        if (p < XR)
            x_load(p, xr[p]);
        if (p < P)
            load_block(p < nb ? p : nb - 1, ring[p]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // 2. tables and the first XB blocks' activations -> LDS
    tb.store_all(tab);
#pragma unroll
    for (int j = 0; j < XB; ++j)
        x_store(j, xr[j]);
    __syncthreads();

    // 3. stream the slice
    f4_t acc[R][MTI][NJ];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int i = 0; i < MTI; ++i)
#pragma unroll
            for (int c = 0; c < NJ; ++c)
                acc[t][i][c] = f4_t{0.f, 0.f, 0.f, 0.f};
    // this lane's fragment addresses within a block slot: chunk
    // (16 h + 4q + jj) ^ xswz(m) of row m, h = j >> 2, jj = j & 3.  Bit 4 of
    // the swizzle only flips the half h, so the second half is the first
    // shifted by hoff = +-16 chunks.
    // xswz depends on the row's low four bits only, so row tile i's
    // addresses are tile 0's plus 512 chunks (16 rows of 32)
    int arow[4], hoff;
    {
        const int f = xswz(r16);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            arow[jj] = r16 * 32 + ((4 * q + jj) ^ (f & 15)) + (f & 16);
        hoff = (f & 16) ? -16 : 16;
    }
    const int glane = (32 * q) >> lg;             // this lane's group offset within a block
    // the slice's last group holding valid k: blocks past the slice and k
    // past K (zero activations) reuse it, so no group index reaches past the
    // tensor's groups (whose padding, for the last channel, lies beyond it)
    const int gmax = (kend - k0 - 1) >> lg;
    // table row of each of this lane's channels, and the element offset of
    // its first group within its scale dwords
    int trow[R], spar[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        trow[t] = (wave * R + t) * 16 + r16;
        spar[t] = tb.parity(trow[t]);
    }

    for (int b0 = 0; b0 < nbp; b0 += U) {
#pragma unroll
        for (int p = 0; p < U; ++p) {
            const int b = b0 + p;
            const int pw = p % P;                 // this block's weight ring slot
            // activation fragments of block b: requested first, so the LDS
            // latency passes while the weights are dequantised
            // (with four row tiles only tile 0's; the others are read as
            // their MFMAs come up)
            constexpr int MTA = MTI > 2 ? 1 : MTI;
            uint4 af[8][MTA];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < MTA; ++i)
                    af[j][i] = xs[b % XSL][arow[j & 3] + (j >> 2) * hoff + 512 * i];
            auto frag = [&](int j, int i) -> uint4 {
                if (i < MTA)
                    return af[j][i];
                return xs[b % XSL][arow[j & 3] + (j >> 2) * hoff + 512 * i];
            };
            // groups of the two pieces (padding blocks clamp to the last group;
            // their activations are zero)
            const int ga = min(((256 * b) >> lg) + glane, gmax);
            const int gb = min(((256 * b + 128) >> lg) + glane, gmax);
            uint32_t words[NW];
            ql::zb_t zb[NW];
            uint32_t s16[R][2];
#pragma unroll
            for (int t = 0; t < R; ++t) {
                const uint16_t* srow = reinterpret_cast<const uint16_t*>(tab + trow[t] * tb.SD);
                const uint32_t* zrow = tab + tb.stot + trow[t] * tb.ZD;
                const uint32_t za_ = (zrow[((g0 + ga) >> 3) - (g0 >> 3)] >> (4 * ((g0 + ga) & 7))) & 0xFu;
                const uint32_t zb_ = (zrow[((g0 + gb) >> 3) - (g0 >> 3)] >> (4 * ((g0 + gb) & 7))) & 0xFu;
                s16[t][0] = srow[spar[t] + ga];
                s16[t][1] = srow[spar[t] + gb];
                const ql::zb_t za = ql::make_zb(za_), zc = ql::make_zb(zb_);
                const uint4 w0 = ring[pw][t][0], w1 = ring[pw][t][1];
                const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    words[8 * t + j] = wv[j];
                    zb[8 * t + j] = j < 4 ? za : zc;
                }
            }
            h8_t bw[NW];
            if constexpr (POST) {
                h2_t d[NW][4];
                ql::dequant_words_qz<NW>(words, zb, d);
#pragma unroll
                for (int j = 0; j < NW; ++j)
                    bw[j] = __builtin_bit_cast(h8_t, make_uint4(ql::h2u(d[j][0]), ql::h2u(d[j][1]),
                                                                ql::h2u(d[j][2]), ql::h2u(d[j][3])));
            } else {
                h2_t s2[NW];
#pragma unroll
                for (int t = 0; t < R; ++t)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        s2[8 * t + j] = ql::scale2(s16[t][j >> 2]);
                ql::dequant_words<NW>(words, zb, s2, bw);
            }
            // Requests for block b + P, in place and in order: activations
            // first, so waiting for them never waits for younger weights.
            // Without the scheduling barriers the compiler sinks and
            // regroups the loads, so waiting for one block means waiting for
            // the whole ring.
            const int nxt = b + P < nb ? b + P : nb - 1;
            __builtin_amdgcn_sched_barrier(0);
            x_load(b + XR, xr[p % XR]);
            load_block(nxt, ring[pw]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (POST) {
#pragma unroll
                for (int t = 0; t < R; ++t) {
                    const float sa = f16_bits_to_f32(s16[t][0]), sb = f16_bits_to_f32(s16[t][1]);
#pragma unroll
                    for (int i = 0; i < MTI; ++i) {
                        f4_t da = f4_t{0.f, 0.f, 0.f, 0.f}, db = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            da = mfma16x16x32(__builtin_bit_cast(h8_t, frag(j, i)), bw[8 * t + j], da);
                            db = mfma16x16x32(__builtin_bit_cast(h8_t, frag(4 + j, i)), bw[8 * t + 4 + j], db);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[t][i][0][r] = __builtin_fmaf(sb, db[r], __builtin_fmaf(sa, da[r], acc[t][i][0][r]));
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < MTI; ++i)
#pragma unroll
                        for (int t = 0; t < R; ++t)
                            acc[t][i][j % NJ] =
                                mfma16x16x32(__builtin_bit_cast(h8_t, frag(j, i)), bw[8 * t + j], acc[t][i][j % NJ]);
            }
            // block b + 1's activations -> the other slot; the barrier
            // publishes them and frees this slot for block b + 2.  Every
            // second block instead (XB = 2): blocks b + 1 and b + 2 into
            // slots last read by blocks b - 3 and b - 2, both before the
            // previous barrier.
            if constexpr (XB == 1) {
                x_store(b + 1, xr[(p + 1) % XR]);
                __syncthreads();
            } else if (p & 1) {
                x_store(b + 1, xr[(p + 1) % XR]);
                x_store(b + 2, xr[(p + 2) % XR]);
                __syncthreads();
            }
        }
    }
    f4_t res[R][MTI];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int i = 0; i < MTI; ++i) {
            if constexpr (NJ == 4)
                res[t][i] = (acc[t][i][0] + acc[t][i][1]) + (acc[t][i][2] + acc[t][i][3]);
            else if constexpr (NJ == 2)
                res[t][i] = acc[t][i][0] + acc[t][i][1];
            else
                res[t][i] = acc[t][i][0];
        }

    if (S == 1) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const int n = n0 + (wave * R + t) * 16 + r16;
#pragma unroll
            for (int i = 0; i < MTI; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = i * 16 + 4 * q + r;
                    if (m < M && n < N)
                        y[(int64_t)m * N + n] = f32_to_f16_bits(res[t][i][r]);
                }
        }
        return;
    }

    if (pair) {
        // two slices: this wave's fragments meet the other slice's in the
        // column block's slots
        f4_t v[R * MTI];
        int row0[R * MTI], col[R * MTI];
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
            for (int i = 0; i < MTI; ++i) {
                v[t * MTI + i] = res[t][i];
                row0[t * MTI + i] = i * 16 + 4 * q;
                col[t * MTI + i] = n0 + (wave * R + t) * 16 + r16;
            }
        pair_finish<R * MTI>(reinterpret_cast<uint64_t*>(part) + ((int64_t)blockIdx.x * T + wave) * (R * MTI * 128),
                             v, row0, col, y, M, N);
        return;
    }

    // 6. split-K: this slice's partial tile with agent-scope stores, then
    //    the arrival and the last arrival's reduction
    float* tile = part + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * (int64_t)M * TW;
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int i = 0; i < MTI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = i * 16 + 4 * q + r;
                if (m < M)
                    __hip_atomic_store(&tile[m * TW + (wave * R + t) * 16 + r16], res[t][i][r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
    splitk_finish<TW>(part, cnt, y, M, N, n0, &s_last);
}

// Loads the compiler does not track, for a register ring that must stay in
// flight across the barrier that publishes LDS: a 16-byte buffer load into
// registers, a 4-byte buffer load into LDS (at M0 + 4 x lane), and a wait
// whose register operands keep each ring entry live, and unread, until its
// load has landed.  Reads past a buffer's end return zero.
typedef uint32_t u4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u4v_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    u4v_t v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(r));
    return v;
}
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds_base)
{
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(off), "s"(r), "{m0}"(lds_base) : "memory");
}
template <int N>
__device__ __forceinline__ void ring_wait(u4v_t& a, u4v_t& b)
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
// the same for a count known only after unrolling (even, at most 30)
__device__ __forceinline__ void ring_wait_n(int n, u4v_t& a, u4v_t& b)
{
    switch (n) {
    case 0: ring_wait<0>(a, b); break;
    case 2: ring_wait<2>(a, b); break;
    case 4: ring_wait<4>(a, b); break;
    case 6: ring_wait<6>(a, b); break;
    case 8: ring_wait<8>(a, b); break;
    case 10: ring_wait<10>(a, b); break;
    case 12: ring_wait<12>(a, b); break;
    case 14: ring_wait<14>(a, b); break;
    case 16: ring_wait<16>(a, b); break;
    case 18: ring_wait<18>(a, b); break;
    case 20: ring_wait<20>(a, b); break;
    case 22: ring_wait<22>(a, b); break;
    case 24: ring_wait<24>(a, b); break;
    case 26: ring_wait<26>(a, b); break;
    case 28: ring_wait<28>(a, b); break;
    default: ring_wait<30>(a, b); break;
    }
}

// ---------------------------------------------------------------------------
// GEMV (m <= 3): one 16-channel tile per workgroup, K split among its KW
// waves, partial sums added through LDS
//
// The decode kernels above give each workgroup several channel tiles and one
// K slice, and sum the slices across workgroups (split-K: each partial tile
// is stored, waited for, counted and re-read).  Timestamps of those launches
// show the weights streaming at the device's copy rate while the blocks are
// consumed, with the time around that loop -- waiting for the tables and
// activations with two weight blocks in flight, and the split-K round trips
// -- costing about as much again.  Here a workgroup owns one tile of 16
// output channels; wave w streams blocks [w nbs / KW, (w + 1) nbs / KW) of the
// workgroup's K range, all of them requested (up to P) before the workgroup
// waits for its tables and activations, and the KW partial sums meet in LDS.
// Launches whose tiles alone would leave CUs unevenly loaded still split K
// across workgroups (gridDim.y slices, summed as in the other decode kernels).
//
// Lane layout (lane l: channel l % 16, quarter q = l / 16, pieces [4q, 4q+4)
// and [16+4q, 16+4q+4) of each 32-word block row), MFMAs, interleaved
// dequantisation and POST scaling: as w4a16_decode_kernel, with M <= MR rows
// (A row r reads activation row min(r, M - 1); output rows >= M are not
// stored; MR = 1 compiles the single-row case without the other rows' work).
// LDS: the scale and zero-point tables of the tile's 16 channels for the
// slice's groups (16 x SD scale dwords from the dword holding the first
// group, 16 x ZD zero words; both padded to whole 64-entry wave loads), the
// slice's activation chunks of each row (reordered in place for the
// interleaved dequantiser, zero past the slice; rows 64 bytes apart in the
// banks), and KW x MR x 16 floats for the sum.
// ---------------------------------------------------------------------------
template <int NB, int P, bool POST, int MR, int KW = 4, int P0 = P>
__global__ __launch_bounds__(64 * KW) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
    const uint32_t* __restrict__ qz, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int m_rows, int N, int K, int lg, int KS, int pair)
{
    static_assert(NB >= 1 && NB <= 16 && P >= 1 && P <= NB, "the ring waits cover up to 16 blocks");
    static_assert(MR >= 1 && MR <= 4, "up to four rows (lanes 0-15 hold output rows 0-3)");
    const int M = MR == 1 ? 1 : m_rows;            // 1 <= M <= MR
    constexpr int TW = 16;
    constexpr int NT = 64 * KW;
    constexpr int NJ = POST ? 1 : 4;               // accumulator chains
    extern __shared__ uint4 gv_lds[];              // 16-byte elements: aligned fragment reads
    uint32_t* const tab = reinterpret_cast<uint32_t*>(gv_lds);
    __shared__ int s_last;

    // this workgroup's K range: balanced 256-k blocks of slice blockIdx.y
    const int nkb = (K + 255) >> 8;
    const int kb_lo = (int)(((int64_t)blockIdx.y * nkb) / gridDim.y);
    const int kb_hi = (int)(((int64_t)(blockIdx.y + 1) * nkb) / gridDim.y);
    const int k0 = kb_lo << 8, kend = min(K, kb_hi << 8);
    const int nch = (kend - k0) >> 3;             // valid activation chunks
    const int nbs = kb_hi - kb_lo;
    const int gs = KS >> lg;                      // groups of the longest slice
    const int g0 = k0 >> lg;
    const int SD = (gs >> 1) + 1, ZD = (gs >> 3) + 2;
    const int stot = TW * SD, ztot = TW * ZD;
    const int spad = (stot + NT - 1) / NT * NT, zpad = (ztot + NT - 1) / NT * NT;   // whole wave loads
    const int CR = KS >> 3;                       // activation chunks stored per row
    const int cpad = (CR + NT - 1) / NT * NT;
    // row stride: whole wave loads plus 4 chunks, so rows sit 64 bytes apart
    // in the LDS banks and the lanes of different rows reading the same chunk
    // do not conflict
    const int CRS = MR == 1 ? cpad : cpad + 4;
    const uint32_t act_off = (uint32_t)(spad + zpad) * 4u;            // bytes, a multiple of 16
    const uint32_t red_off = act_off + (uint32_t)(M * CRS) * 16u;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * TW;
    const int KWD = K >> 3, NG = K >> lg, ZW = (NG + 7) >> 3;
    const int wb0 = (wave * nbs) / KW, nb = ((wave + 1) * nbs) / KW - wb0;   // this wave's blocks
    const uint32_t lds0 = (uint32_t)(uintptr_t)tab;

    // 1. requests, oldest first: tables and activations straight to LDS,
    //    then this wave's first P weight blocks (blocks past its range re-read
    //    its last block, so 2 P loads always follow the others)
    {
        const uint32_t sbytes = ((uint32_t)N * (uint32_t)NG * 2u + 3u) & ~3u;
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(sc, sbytes);
        const __amdgpu_buffer_rsrc_t rzr = make_rsrc(qz, (uint32_t)N * (uint32_t)ZW * 4u);
        for (int u = 0; u < spad; u += NT) {
            const int e = min(u + tid, stot - 1);
            const int rr = e / SD, col = e - rr * SD;
            const uint32_t row = (uint32_t)min(n0 + rr, N - 1);
            const uint32_t dw = min(((row * (uint32_t)NG + (uint32_t)g0) >> 1) + (uint32_t)col, sbytes / 4u - 1u);
            buf_dma4(rsc, dw * 4u, (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(u + wave * 64) * 4u));
        }
        for (int u = 0; u < zpad; u += NT) {
            const int e = min(u + tid, ztot - 1);
            const int rr = e / ZD, col = e - rr * ZD;
            const uint32_t row = (uint32_t)min(n0 + rr, N - 1);
            const uint32_t wd = min(row * (uint32_t)ZW + (uint32_t)(g0 >> 3) + (uint32_t)col,
                                    (uint32_t)N * (uint32_t)ZW - 1u);
            buf_dma4(rzr, wd * 4u,
                     (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(spad + u + wave * 64) * 4u));
        }
        for (int r = 0; r < M; ++r)
            for (int u = 0; u < cpad; u += NT) {
                const int c = min(u + tid, nch - 1);
                ql::dma16s(x, (uint32_t)(r * K + k0 + 8 * c) * 2u,
                           (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + act_off +
                                                                    (uint32_t)(r * CRS + u + wave * 64) * 16u));
            }
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * (uint32_t)KWD * 4u);
    const int nrow = min(n0 + r16, N - 1);
    const int last = nb > 0 ? nb - 1 : 0;
    const uint32_t ow = (uint32_t)nrow * (uint32_t)KWD * 4u + (uint32_t)(k0 + 256 * wb0 + 32 * q) / 2u;
    u4v_t ring[P][2];
#pragma unroll
    for (int b = 0; b < P0; ++b) {
        const uint32_t bw = ow + (uint32_t)min(b, last) * 128u;
        ring[b][0] = buf_load16(rw, bw);
        ring[b][1] = buf_load16(rw, bw + 64u);
    }
    // 2. wait for everything but those weights and publish the tables and
    //    the activations (the chunks past the slice's end hold copies of its
    //    last chunk; the blocks that read them are masked below), then
    //    request the rest of the ring: issued after the small loads, the
    //    weight stream does not delay them
    ql::stage_barrier<2 * P0>();
#pragma unroll
    for (int b = P0; b < P; ++b) {
        const uint32_t bw = ow + (uint32_t)min(b, last) * 128u;
        ring[b][0] = buf_load16(rw, bw);
        ring[b][1] = buf_load16(rw, bw + 64u);
    }
    // 3. each activation chunk, once: reordered for the interleaved
    //    dequantiser (13 operations per weight word instead of 16 in natural
    //    order, which the block loop's issue rate feels), or cleared past the
    //    slice's end
    {
        for (int r = 0; r < M; ++r) {
            uint4* xw = gv_lds + act_off / 16 + r * CRS;
            for (int e = tid; e < CR; e += NT) {
                const bool ok = e < nch;
                xw[e] = ql::permute_x8_sel(xw[e], ok ? ql::kPermLo : ql::kPermZero, ok ? ql::kPermHi : ql::kPermZero);
            }
        }
        __syncthreads();
    }

    // 4. this wave's blocks
    const uint4* xs = gv_lds + act_off / 16 + min(r16, M - 1) * CRS;   // this lane's A row
    const int glane = (32 * q) >> lg;
    // the slice's last group holding valid k: blocks past the slice and k
    // past K (zero activations) reuse it, so no group index reaches past the
    // tensor's groups (whose padding, for the last channel, lies beyond it)
    const int gmax = (kend - k0 - 1) >> lg;
    const int spar = (int)(((uint32_t)nrow * (uint32_t)NG + (uint32_t)g0) & 1u);
    const uint16_t* srow = reinterpret_cast<const uint16_t*>(tab + r16 * SD);
    const uint32_t* zrow = tab + spad + r16 * ZD;
    f4_t acc[NJ];
#pragma unroll
    for (int c = 0; c < NJ; ++c)
        acc[c] = f4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        constexpr int kLast = NB - 1;
        u4v_t(&rs)[2] = ring[b % P];
        ring_wait_n(2 * ((b + P - 1 <= kLast ? b + P - 1 : kLast) - b), rs[0], rs[1]);
        if (b >= nb) {
            if (b + P < NB) {
                const uint32_t bw = ow + (uint32_t)last * 128u;
                rs[0] = buf_load16(rw, bw);
                rs[1] = buf_load16(rw, bw + 64u);
            }
            continue;
        }
        const int bb = wb0 + b;                   // block within the slice
        uint4 af[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            af[j] = xs[32 * bb + 16 * (j >> 2) + 4 * q + (j & 3)];
        const int ga = min(((256 * bb) >> lg) + glane, gmax);
        const int gb = min(((256 * bb + 128) >> lg) + glane, gmax);
        const uint32_t za_ = (zrow[((g0 + ga) >> 3) - (g0 >> 3)] >> (4 * ((g0 + ga) & 7))) & 0xFu;
        const uint32_t zb_ = (zrow[((g0 + gb) >> 3) - (g0 >> 3)] >> (4 * ((g0 + gb) & 7))) & 0xFu;
        const uint32_t s16a = srow[spar + ga], s16b = srow[spar + gb];
        const ql::zb_t za = ql::make_zb(za_), zc = ql::make_zb(zb_);
        const u4v_t w0 = rs[0], w1 = rs[1];
        const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        // the slot's next block, once its words are read
        if (b + P < NB) {
            const uint32_t bw = ow + (uint32_t)min(b + P, last) * 128u;
            rs[0] = buf_load16(rw, bw);
            rs[1] = buf_load16(rw, bw + 64u);
        }
        ql::zb_t zb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            zb[j] = j < 4 ? za : zc;
        h8_t bw[8];
        if constexpr (POST) {
            h2_t d[8][4];
            ql::dequant_words_qz<8>(words, zb, d);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                bw[j] = __builtin_bit_cast(h8_t, make_uint4(ql::h2u(d[j][0]), ql::h2u(d[j][1]), ql::h2u(d[j][2]),
                                                            ql::h2u(d[j][3])));
            const float sa = f16_bits_to_f32(s16a), sb = f16_bits_to_f32(s16b);
            f4_t da = f4_t{0.f, 0.f, 0.f, 0.f}, db = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                da = mfma16x16x32(__builtin_bit_cast(h8_t, af[j]), bw[j], da);
                db = mfma16x16x32(__builtin_bit_cast(h8_t, af[4 + j]), bw[4 + j], db);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[0][r] = __builtin_fmaf(sb, db[r], __builtin_fmaf(sa, da[r], acc[0][r]));
        } else {
            h2_t s2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s2[j] = ql::scale2(j < 4 ? s16a : s16b);
            ql::dequant_words<8>(words, zb, s2, bw);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j % NJ] = mfma16x16x32(__builtin_bit_cast(h8_t, af[j]), bw[j], acc[j % NJ]);
        }
    }
    f4_t res;
    if constexpr (NJ == 4)
        res = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    else
        res = acc[0];

    // 5. the waves' partial tiles of output rows 0 .. M-1 (lanes 0-15 hold
    //    rows 0-3) meet in LDS and are added in wave order
    float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(gv_lds) + red_off);
    if (q == 0) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
            if (r < M)
                red[(wave * MR + r) * TW + r16] = res[r];
    }
    __syncthreads();
    const int rr = tid >> 4, cc = tid & 15;       // output row and channel of this thread
    float sum = 0.0f;
    if (rr < M) {
#pragma unroll
        for (int w = 0; w < KW; ++w)
            sum += red[(w * MR + rr) * TW + cc];
    }
    const int ncol = n0 + cc;
    if (gridDim.y == 1) {
        if (rr < M && ncol < N)
            y[(int64_t)rr * N + ncol] = f32_to_f16_bits(sum);
        return;
    }
    if (pair) {
        // two slices: each output meets the other slice's partial in one
        // 4-byte slot, [column block][MR rows][16 channels]
        if (rr < M)
            pair_finish_one(reinterpret_cast<uint32_t*>(part) + ((int64_t)blockIdx.x * MR + rr) * TW + cc, sum,
                            y, rr, ncol, N);
        return;
    }
    // 6. split-K across workgroups: this slice's M x 16 partial tile, then
    //    the arrival and the last arrival's reduction
    float* tile = part + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * (int64_t)(M * TW);
    if (rr < M)
        __hip_atomic_store(&tile[rr * TW + cc], sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    splitk_finish<TW>(part, cnt, y, M, N, n0, &s_last);
}

// ---------------------------------------------------------------------------
// GEMM (m > 64): block tile BM x BN, K advanced in tiles of 64, 4 waves as
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
                const ql::zb_t zb1 = ql::make_zb(rz[u] & 0xFu);
                const h2_t s21 = ql::scale2(rs[u]);
                const uint32_t words[4] = {rb[u].x, rb[u].y, rb[u].z, rb[u].w};
                const ql::zb_t zb[4] = {zb1, zb1, zb1, zb1};
                const h2_t s2[4] = {s21, s21, s21, s21};
                h8_t wv[4];
                ql::dequant_words<4>(words, zb, s2, wv);
                uint8_t* dst = Bs + buf * BN * kGRow + row * kGRow + (c & 1) * 64;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<h8_t*>(dst + j * 16) = wv[j];
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
// Split-K completion of a GEMM tile, after this thread's agent-scope stores
// of its part of the tile's fp32 partial sums ([rows][BN] at
// part[(slice * tiles + tile) * srows * BN], srows = min(M, BM)): wait for
// them, arrive on the tile's counter, and if this workgroup arrived last, sum
// the nsl partial tiles in slice order and store y.  As splitk_finish: every
// cross-workgroup value moves through agent-scope accesses, the last arrival
// resets the counter, and the order of the sum does not depend on timing.
template <int BN>
__device__ __forceinline__ void gemm_splitk_finish(float* __restrict__ part, uint32_t* __restrict__ cnt,
                                                   uint16_t* __restrict__ y, int M, int N, int m0, int n0, int tile,
                                                   int tiles, int nsl, int srows, int* s_last)
{
    const int tid = threadIdx.x;
    __builtin_amdgcn_s_waitcnt(0);      // this thread's partial stores have completed
    __syncthreads();                    // ... and so have every other thread's
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (prev == (uint32_t)(nsl - 1));
    }
    __syncthreads();
    if (!*s_last)
        return;
    const uint32_t tile_bytes = (uint32_t)srows * BN * 4u;
    const uint32_t slice_bytes = (uint32_t)tiles * tile_bytes;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, (uint32_t)nsl * slice_bytes);
    constexpr int kSc1 = 16;            // cache policy: agent scope (bypasses this CU's L1)
    const int rows = min(srows, M - m0);
    for (int v = tid; v < rows * (BN / 4); v += blockDim.x) {
        const uint32_t off = (uint32_t)tile * tile_bytes + (uint32_t)v * 16u;
        f4_t sum = f4_t{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nsl; s0 += 8) {
            f4_t pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sl = min(s0 + u, nsl - 1);
                pv[u] = __builtin_bit_cast(
                    f4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (int)(off + (uint32_t)sl * slice_bytes), 0, kSc1));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < nsl)
                    sum += pv[u];
        }
        const int m = m0 + v / (BN / 4), nn = n0 + (v % (BN / 4)) * 4;
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
    if (tid == 0)
        __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BM_, int BN_, int WM_, int S_, int GM_, int NW_ = 4, int KG_ = 1>
struct W4PipeCfg {
    static constexpr int BM = BM_, BN = BN_, S = S_, GM = GM_;
    static constexpr int NW = NW_;                     // waves; the first 4 issue the ring loads
    static constexpr int KG = KG_;                     // wave groups splitting each block's k steps
    static constexpr int WM = WM_, WN = NW_ / (WM_ * KG_);   // waves along m and n (per group)
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
    static_assert(WM * WN * KG == NW && (NW == 4 || NW == 8) && (KG == 1 || KG == 2) && BM % (16 * WM) == 0 &&
                      BN % (16 * WN) == 0 && BN % 64 == 0,
                  "4 or 8 waves of 16-row fragments, 64-row tables");
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


// The same for MFMAs that each read one A fragment in turn (FJ MFMAs per
// fragment, then that fragment's refill from LDS), V vector-ALU instructions
// after each MFMA.
template <int FI, int FJ, int V>
__device__ __forceinline__ void interleave_rolling()
{
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // vector ALU
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
    }
}

template <class C>
__global__ __launch_bounds__(C::NW * 64) void w4a16_gemm_pipe_kernel(const uint16_t* __restrict__ x,
                                                              const uint32_t* __restrict__ qw,
                                                              const uint16_t* __restrict__ sc,
                                                              const uint32_t* __restrict__ qz,
                                                              uint16_t* __restrict__ y, int M, int N, int K, int lg,
                                                              float* __restrict__ part, uint32_t* __restrict__ cnt,
                                                              int KB, int nsl)
{
    constexpr int BM = C::BM, BN = C::BN, S = C::S, D = C::D, DA = C::DA, DB = C::DB;
    constexpr int TM = BM / C::WM, TN = BN / C::WN;
    constexpr int FI = TM / 16, FJ = TN / 16;
    constexpr int U = S % 2 == 0 ? S : 2 * S;          // unrolled blocks: slot and register parity static
    static_assert(S >= 2 && D * (S - 1) < 64, "ring depth within vmcnt");
    extern __shared__ __attribute__((aligned(1024))) uint8_t pl[];   // S * kStageBytes

    // Work unit u = slice * tiles + tile (split-K: nsl slices of KB blocks of
    // 128 k; nsl = 1 without), so the units one XCD runs share a K slice of
    // the activations.
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int tiles = tm * tn;
    const int unit = xcd_tile(blockIdx.x, tiles * nsl);
    if (unit >= tiles * nsl)
        return;
    const int slice = unit / tiles, tile = unit - slice * tiles;
    const int gsz = C::GM * tn;                        // tiles per group of GM m-tiles
    const int grp = tile / gsz, first = grp * C::GM;
    const int gm = min(tm - first, C::GM);
    const int m0 = (first + (tile - grp * gsz) % gm) * BM;
    const int n0 = ((tile - grp * gsz) / gm) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // k group kg takes steps [s0, s0 + NS) of every block; within a group,
    // wave wl owns sub-tile (wm, wn)
    constexpr int NS = 4 / C::KG;
    const int kg = wave / (C::WM * C::WN), wl = wave % (C::WM * C::WN);
    const int wm = wl / C::WN, wn = wl % C::WN;
    const int s0 = kg * NS;
    const int q = lane >> 4, r16 = lane & 15;
    const uint32_t lds0 = (uint32_t)(uintptr_t)pl;
    const int NG = K >> lg, ZW = (NG + 7) >> 3;
    const int gsh = lg - 4;                            // block kb's first group is kb << (7 - lg)

    // Ring loads of this wave (waves 0-3 issue them all; with 8 waves, waves
    // 4-7 only compute, and their waits for the ring are trivially met).
    // Activations: 1 KiB = 4 rows of 256 bytes,
    // lane l writes physical chunk l % 16 of row l / 16.  Weights: 1 KiB =
    // 16 rows of 64 bytes, lane l writes physical chunk l % 4 of row l / 4.
    // Tables: 64 rows of 4 bytes per load; load t (of 4 * BN/64, spread over
    // the waves) is zero words (t / kDwRows == 0), scale dword 0 (1), scale
    // dword 1 (2, G = 32 only, else a repeat of dword 0) or a repeat of the
    // zero words (3).  Rows past M or N re-read the last row (never stored).
    // Each load's per-lane source is a 32-bit byte offset from its tensor
    // (the host sends tensors of 4 GiB or more to the register-staged kernel).
    uint32_t soff[D];
    uint32_t tdst[D - DA - DB];                        // LDS offsets of the table loads
    bool tscale[D - DA - DB];                          // scale dwords (else zero words)
    // loading wave, in a scalar register: every ring load's LDS destination
    // is then formed by scalar instructions
    const int lw = __builtin_amdgcn_readfirstlane(wave & 3);
#pragma unroll
    for (int u = 0; u < D; ++u) {
        if (u < DA) {
            const int blk = lw + 4 * u;
            const int row = blk * 4 + (lane >> 4);
            const int c = (lane & 15) ^ ql::swz256(row);
            const int m = min(m0 + row, M - 1);
            soff[u] = (uint32_t)m * (uint32_t)K * 2u + 16u * (uint32_t)c;
        } else if (u < DA + DB) {
            const int blk = lw + 4 * (u - DA);
            const int row = blk * 16 + (lane >> 2);
            const int c = (lane & 3) ^ ql::swz64(row);
            const int n = min(n0 + row, N - 1);
            soff[u] = (uint32_t)n * (uint32_t)(K / 2) + 16u * (uint32_t)c;
        } else {
            const int t = lw + 4 * (u - DA - DB);
            const int kind = t / C::kDwRows, part = t % C::kDwRows;
            const int row = 64 * part + lane;
            const int n = min(n0 + row, N - 1);
            tscale[u - DA - DB] = kind == 1 || kind == 2;
            if (kind == 1 || kind == 2) {
                const int extra = (kind == 2 && lg == 5) ? 4 : 0;
                soff[u] = (uint32_t)n * (uint32_t)NG * 2u + (uint32_t)extra;
                tdst[u - DA - DB] = (uint32_t)(C::kSoff + (kind == 2 ? 4 * BN : 0) + 4 * 64 * part);
            } else {
                soff[u] = (uint32_t)n * (uint32_t)ZW * 4u;
                tdst[u - DA - DB] = (uint32_t)(C::kZoff + 4 * 64 * part);
            }
        }
    }
    auto issue = [&](int kb, int slot) {
        if (C::NW > 4 && wave >= 4)
            return;
        const uint32_t sbase = lds0 + slot * C::kStageBytes;
        // scale byte offset of block kb: first group * 2, aligned down to 4
        const int sofs = ((kb << (7 - lg)) * 2) & ~3;
        const int zofs = 4 * (kb >> gsh);
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (u < DA) {
                ql::dma16s(reinterpret_cast<const uint8_t*>(x) + (int64_t)kb * 256, soff[u],
                           (uint32_t)__builtin_amdgcn_readfirstlane(sbase + (uint32_t)((lw + 4 * u) * 1024)));
            } else if (u < DA + DB) {
                ql::dma16s(reinterpret_cast<const uint8_t*>(qw) + (int64_t)kb * 64, soff[u],
                           (uint32_t)__builtin_amdgcn_readfirstlane(
                               sbase + (uint32_t)(C::kAbytes + (lw + 4 * (u - DA)) * 1024)));
            } else {
                // 64 rows x 4 bytes, lane l -> row 64 * part + l; the table
                // kind is the same for the whole wave
                const bool ts = __builtin_amdgcn_readfirstlane((int)tscale[u - DA - DB]) != 0;
                const uint8_t* b = ts ? reinterpret_cast<const uint8_t*>(sc) + sofs
                                      : reinterpret_cast<const uint8_t*>(qz) + zofs;
                ql::dma4s(b, soff[u], (uint32_t)__builtin_amdgcn_readfirstlane(sbase + tdst[u - DA - DB]));
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
            const uint8_t* wp = base + C::kAbytes + r * C::kBrow + 16 * (q ^ ql::swz64(r));
            if constexpr (C::KG == 2) {
                // this group's words 4q + s0 and 4q + s0 + 1 of the chunk
                const uint2 h = *reinterpret_cast<const uint2*>(wp + 4 * s0);
                fb[j] = make_uint4(h.x, h.y, 0u, 0u);
            } else {
                fb[j] = *reinterpret_cast<const uint4*>(wp);
            }
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

    uint4 fa[C::KG == 2 ? 1 : 2][FI], fb[2][FJ];
    uint32_t zr[2][FJ], sr[2][FJ];
    ql::zb_t zb[2][FJ];
    h2_t s2[2][FJ];
    h8_t bw[2][FJ];
    const int kb_lo = slice * KB;                      // this slice's blocks [kb_lo, kb_hi)
    const int kb_hi = min(K / 128, kb_lo + KB);
    const int nkl = kb_hi - kb_lo;
    auto word = [](const uint4& w4, int st) { return st == 0 ? w4.x : st == 1 ? w4.y : st == 2 ? w4.z : w4.w; };
    // zero bias and scale of block kb from its table words
    auto set_zs = [&](int kb, int p) {
        const int zsh = 4 * (((kb * 128 + 32 * q) >> lg) & 7);
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            zb[p][j] = ql::make_zb((zr[p][j] >> zsh) & 0xFu);
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
        issue(kb_lo + (s < nkl ? s : nkl - 1), s);
    ql::stage_barrier<D * (S - 1)>();   // the slice's first block landed
    read_a(0, s0, fa[0]);
    read_b(0, kb_lo, fb[0], zr[0], sr[0]);
    set_zs(kb_lo, 0);
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
        for (int st = 0; st < NS; ++st) {
            const int cur = st & 1;
            if (st < NS - 1) {
                read_a(slot, s0 + st + 1, fa[cur ^ 1]);
                dequant(par, st + 1, bw[cur ^ 1]);
                mfmas(cur, 0, FI);
                interleave<FI, FI * FJ, 3>();
            } else {
                ql::stage_barrier<D * (S - 2)>();
                issue(min(kb + S, kb_hi - 1), slot);
                read_b((u + 1) % S, kb + 1, fb[par ^ 1], zr[par ^ 1], sr[par ^ 1]);
                read_a((u + 1) % S, s0, fa[cur ^ 1]);
                mfmas(cur, 0, FI / 2);
                set_zs(kb + 1, par ^ 1);
                dequant(par ^ 1, 0, bw[cur ^ 1]);
                mfmas(cur, FI / 2, FI);
                interleave<FI + 3 * FJ, FI * FJ, 3>();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Two k groups (NS = 2 steps per block and wave): one buffer of A
    // fragments, each refilled with the next step's fragment right after the
    // MFMAs that read it, so a wave holds FI fragments instead of 2 FI.
    auto read_a1 = [&](int slot, int st, int i) -> uint4 {
        const uint8_t* base = pl + slot * C::kStageBytes;
        const int r = wm * TM + 16 * i + r16;
        return *reinterpret_cast<const uint4*>(base + r * C::kArow + 16 * ((4 * q + st) ^ ql::swz256(r)));
    };
    auto block_k2 = [&](int kb, int u) {
        const int slot = u % S, par = u & 1;
        // step s0: A fragments of step s0 in fa[0], weights in bw[0]
#pragma unroll
        for (int i = 0; i < FI; ++i) {
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = mfma16x16x32(bw[0][j], __builtin_bit_cast(h8_t, fa[0][i]), acc[i][j]);
            fa[0][i] = read_a1(slot, s0 + 1, i);
        }
        dequant(par, 1, bw[1]);
        interleave_rolling<FI, FJ, 2>();
        __builtin_amdgcn_sched_barrier(0);
        // step s0 + 1: wait for the next block, refill this block's slot, read
        // the next block's weights and tables, then its step-s0 A fragments
        ql::stage_barrier<D * (S - 2)>();
        issue(min(kb + S, kb_hi - 1), slot);
        read_b((u + 1) % S, kb + 1, fb[par ^ 1], zr[par ^ 1], sr[par ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FI; ++i) {
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = mfma16x16x32(bw[1][j], __builtin_bit_cast(h8_t, fa[0][i]), acc[i][j]);
            fa[0][i] = read_a1((u + 1) % S, s0, i);
        }
        set_zs(kb + 1, par ^ 1);
        dequant(par ^ 1, 0, bw[0]);
        interleave_rolling<FI, FJ, 2>();
        __builtin_amdgcn_sched_barrier(0);
    };
    int kb0 = 0;
    for (; kb0 + U <= nkl; kb0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (C::KG == 2)
                block_k2(kb_lo + kb0 + u, u);
            else
                block(kb_lo + kb0 + u, u);
        }
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (kb0 + u < nkl) {
            if constexpr (C::KG == 2)
                block_k2(kb_lo + kb0 + u, u);
            else
                block(kb_lo + kb0 + u, u);
        }
    ql::stage_barrier<0>();   // drain the trailing reloads; the ring's LDS is free from here

    if constexpr (C::KG == 2) {
        // group 1 hands its partial sums to group 0 through LDS (lane-major,
        // 256 bytes per accumulator element and wave); group 0 adds them in
        // a fixed order and alone stores the tile
        float* red = reinterpret_cast<float*>(pl);
        static_assert(C::WM * C::WN * FI * FJ * 4 * 64 * 4 <= C::kLds, "reduction fits in the ring's LDS");
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[(((wl * FI + i) * FJ + j) * 4 + r) * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][r] += red[(((wl * FI + i) * FJ + j) * 4 + r) * 64 + lane];
        }
        __syncthreads();
    }
    const bool storer = kg == 0;

    if (nsl > 1) {
        // this slice's partial tile (rows < M), then the split-K completion;
        // the first LDS word serves as the workgroup's flag
        const int srows = M < BM ? M : BM;
        float* tp = part + ((int64_t)slice * tiles + tile) * (int64_t)srows * BN;
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int ml = wm * TM + i * 16 + r16;
                const int nl = wn * TN + j * 16 + 4 * q;
                if (storer && m0 + ml < M)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __hip_atomic_store(&tp[ml * BN + nl + r], acc[i][j][r], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        gemm_splitk_finish<BN>(part, cnt, y, M, N, m0, n0, tile, tiles, nsl, srows, reinterpret_cast<int*>(pl));
        return;
    }

    if (!storer)
        return;
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
    bool gemv;  // GEMV kernel, m <= 3 (one 16-channel tile per workgroup; else the streamed one)
    int mt;     // 16, 32 or 64
    int t;      // waves per workgroup (streamed kernel: 4 or 6)
    int r;      // 16-channel tiles per wave
    int p;      // blocks in flight per wave (GEMV kernel: most blocks per wave)
    bool post;  // group scale applied to the fp32 MFMA result (128-channel groups)
    int ks;     // k per slice (multiple of 256)
    int slices; // split-K factor
    int nblk;   // column blocks
    bool pair;  // two slices that meet in exchange slots (no counters, no partial tiles)
    size_t lds_bytes;   // dynamic LDS bytes
    size_t part_offset, part_bytes;
};

// The workspace starts with a fixed region that is zero between calls: the
// arrival counters, then the two-slice exchange slots; partial sums follow
// it.  A fixed region keeps calls of different shapes from reading each
// other's partial sums as counters or slots when they share one workspace.
constexpr size_t kCounterBytes = 32768;
constexpr size_t kPairBytes = (size_t)4 << 20;
constexpr size_t kFixedBytes = kCounterBytes + kPairBytes;
static_assert(kFixedBytes == QL_W4A16_WS_ZERO_BYTES, "the header states the fixed region's size");
constexpr int kMaxDecodeBlocks = (int)(kCounterBytes / sizeof(uint32_t));
constexpr int kDecodeWaveMin = 1024;             // 4 streaming waves per CU (MI355X: 256 CUs)
constexpr int kDecodeWaveTarget = 2048;          // 8 streaming waves per CU
constexpr bool kDecodeWide = true;               // six-wave workgroups where they avoid doubled CUs
constexpr int64_t kDecodeMaxRows = 64;           // the decode path takes m <= 64

// Dynamic LDS of the decode kernel: the scale and zero-point tables.
size_t decode_tables(int64_t sblocks, int64_t channels, int group)
{
    const int64_t gs = sblocks * 256 / group;
    return (size_t)channels * (size_t)((gs >> 1) + 1 + (gs >> 3) + 2) * 4;
}
// Tile and split choice (measured on the MLP decode shapes).  K is split
// until the launch has ~8 streaming waves per CU, except that from 9 rows on
// a launch whose column tiles alone give >= 4 waves per CU is not split: there
// the partial sums (which grow with m) cost more than the extra waves gain.
DecodePlan decode_plan(int64_t m, int64_t n, int64_t k, int group)
{
    DecodePlan p{};
    p.mt = m <= 16 ? 16 : (m <= 32 ? 32 : 64);
    p.p = 2;
    p.r = 1;
    p.post = group == 128;
    p.t = p.mt == 64 ? 8 : 4;
    const int64_t cus = ql::cu_count();
    // From 9 rows on, a launch not split along K whose four-wave column
    // blocks would put two workgroups on some CUs, while six-wave ones fit
    // one per CU, takes six-wave workgroups: the busiest CU then holds six
    // channel tiles instead of eight.
    if (kDecodeWide && p.mt < 64 && m > 8 && cus > 0 && (n + 63) / 64 > cus && (n + 95) / 96 <= cus &&
        (n + 63) / 64 * 4 >= kDecodeWaveMin)
        p.t = 6;
    const int64_t tw = 16 * p.t * p.r;
    p.nblk = (int)((n + tw - 1) / tw);
    const int64_t kblocks = (k + 255) / 256;
    const int64_t waves = (int64_t)p.nblk * p.t;
    const int64_t target = (m > 8 && (waves >= kDecodeWaveMin || p.t == 6)) ? waves : kDecodeWaveTarget;
    int64_t slices = std::min<int64_t>((target + waves - 1) / waves, kblocks);
    // Two slices meet in exchange slots (one atomic round trip) where more
    // need the counter protocol (three dependent round trips, about 1 us
    // more): where that balance asks for three or four slices, two are as
    // fast or faster (measured at M = 4-32, N = 8192-14336 and the 13B up
    // projection: 1.1-4.4 us less at three slices, even at four).  Not for
    // the 64-row kernel, whose eight exchanges per lane cost more than the
    // counter protocol (13B up M = 64: 29.6 against 26.0 us).
    const size_t pair_slots = (size_t)p.nblk * (size_t)(tw / 16) * (size_t)(p.mt / 16) * 1024;
    const bool pair_ok = p.mt <= 32 && pair_slots <= kPairBytes;
    if ((slices == 3 || slices == 4) && pair_ok)
        slices = 2;
    // 64-row workgroups run one per CU: no more slices than keep the launch
    // in one round
    if (p.mt == 64 && cus > 0)
        slices = std::max<int64_t>(1, std::min<int64_t>(slices, cus / p.nblk));
    const int64_t sblocks = (kblocks + slices - 1) / slices;   // the longest balanced slice
    p.ks = (int)(sblocks * 256);
    p.lds_bytes = decode_tables(sblocks, tw, group);
    p.slices = (int)slices;
    p.part_offset = kFixedBytes;
    // two slices: 8-byte slots for pairs of output rows, [nblk][tw / 16][mt / 16][64 lanes][2]
    p.pair = p.slices == 2 && pair_ok;
    // else partial tiles [slices][nblk][m][tw] fp32
    p.part_bytes = p.slices > 1 && !p.pair ? (size_t)p.slices * (size_t)p.nblk * (size_t)m * (size_t)tw * sizeof(float) : 0;
    return p;
}

// GEMV plan (m <= kGemvMaxRows): one workgroup of kGemvWaves waves per
// 16-channel tile; K split across workgroups (sg slices) only where that
// evens out the load per CU by more than the cross-workgroup sum costs, or
// where the slice's activation rows would not fit their budget.  The costs
// are fitted to the LLaMA-7B and 13B shapes: with 128-channel groups 5% for
// two slices, which meet in exchange slots, and 30% for more (13B down M = 1
// 12.9 us at two slices against 13.7 us at four); with smaller groups 10% and
// 15% (13B down M = 1 at G = 32: 17.2 us at two slices, 15.8 at four).
constexpr int kGemvWaves = 4;
constexpr int kGemvEarlyBlocks = 2;              // weight blocks requested before the tables and activations land
constexpr int kGemvMaxWaveBlocks = 16;
constexpr int64_t kGemvMaxActBytes = 98304;
constexpr int kGemvMaxRows = 3;
constexpr int kGemvResidentWgs = 8;              // four-wave workgroups per CU at most (32 waves)

DecodePlan decode_plan_gemv(int64_t m, int64_t n, int64_t k, int group)
{
    DecodePlan p{};
    p.gemv = true;
    p.mt = 16;
    p.post = group == 128;
    p.nblk = (int)((n + 15) / 16);
    const int64_t kblocks = (k + 255) / 256;
    int64_t sg_min = 1;
    while ((kblocks + sg_min - 1) / sg_min > (int64_t)kGemvWaves * kGemvMaxWaveBlocks ||
           (kblocks + sg_min - 1) / sg_min * 512 * m > kGemvMaxActBytes)
        ++sg_min;
    int64_t sg = sg_min;
    const int64_t cus = ql::cu_count();
    if (cus > 0) {
        double best = 1e30;
        for (int64_t s2 = sg_min; s2 <= std::min<int64_t>(4 * sg_min, kblocks); ++s2) {
            // two slices meet in exchange slots, more through the counter
            // protocol; two are not taken where their workgroups would
            // not all be resident at once
            if (s2 == 2 && p.nblk * 2 > kGemvResidentWgs * cus)
                continue;
            const double cost = s2 == 1 ? 1.0 : (p.post ? (s2 == 2 ? 1.05 : 1.3) : (s2 == 2 ? 1.1 : 1.15));
            const double load = (double)((p.nblk * s2 + cus - 1) / cus) / (double)s2 * cost;
            if (load < best - 1e-9) {
                best = load;
                sg = s2;
            }
        }
    }
    p.slices = (int)sg;
    const int64_t sblocks = (kblocks + sg - 1) / sg;               // the longest slice
    p.ks = (int)(sblocks * 256);
    const int64_t wave_blocks = (sblocks + kGemvWaves - 1) / kGemvWaves;
    p.p = wave_blocks <= 4 ? 4 : (wave_blocks <= 8 ? 8 : 16);      // blocks unrolled per wave
    // LDS: the kernel's layout (tables padded to whole wave loads, the
    // activation chunks, the partial sums)
    const int64_t nt = 64 * kGemvWaves;
    const int64_t gs = (int64_t)p.ks / group;
    const int64_t stot = 16 * ((gs >> 1) + 1), ztot = 16 * ((gs >> 3) + 2);
    const int64_t spad = (stot + nt - 1) / nt * nt, zpad = (ztot + nt - 1) / nt * nt;
    const int64_t cpad = (p.ks / 8 + nt - 1) / nt * nt;
    const int64_t mr = m > 1 ? kGemvMaxRows : 1;
    p.lds_bytes = (size_t)((spad + zpad) * 4 + m * (cpad + (m > 1 ? 4 : 0)) * 16 + kGemvWaves * mr * 16 * 4);
    p.part_offset = kFixedBytes;
    // two slices: 4-byte slots [nblk][rows][16]; else partial tiles [slices][nblk][m][16] fp32
    p.pair = p.slices == 2 && (size_t)p.nblk * (size_t)kGemvMaxRows * 16 * sizeof(float) <= kPairBytes;
    p.part_bytes = p.slices > 1 && !p.pair ? (size_t)p.slices * (size_t)p.nblk * (size_t)m * 16 * sizeof(float) : 0;
    return p;
}

// Kernel choice by m (measured on the MLP decode shapes).  Two or three rows
// on a wide layer, where the streamed kernel splits K in two exchanging
// slices, take the streamed kernel (gate/up M = 2 / 3 13.7 / 14.1 us against
// 13.8 / 14.8 for the GEMV, 13B up 12.9 / 13.0 against 13.9 / 14.7); on
// narrow layers, where it would split K eight ways, the GEMV stays (down
// M = 2 / 3 10.3 / 10.9 against 11.2, q_proj 5.2 / 5.4 against 8.4).
DecodePlan decode_plan_auto(int64_t m, int64_t n, int64_t k, int group)
{
    if (m <= kGemvMaxRows) {
        if (m >= 2) {
            DecodePlan s = decode_plan(m, n, k, group);
            if (s.pair)
                return s;
        }
        DecodePlan p = decode_plan_gemv(m, n, k, group);
        if (ql::lds_fits(p.lds_bytes))
            return p;
    }
    return decode_plan(m, n, k, group);
}

size_t decode_workspace(const DecodePlan& p) { return p.slices > 1 ? p.part_offset + p.part_bytes : 0; }

// GEMM path (any m): tile shape, ring kernel or register-staged kernel, and
// the split-K factor.  Launches whose tiles would leave CUs idle (few tiles:
// small m or small n) split K into nsl slices of kb 128-blocks, so that
// tiles x nsl fills the CUs; partial tiles are summed by the last arrival as
// in the decode path.
constexpr int kGemmMinSliceBlocks = 4;           // no slice shorter than 512 k
constexpr bool kGemmKGroups = true;              // one-round launches: 8 waves in two k groups

struct GemmPlan {
    bool pipe;      // LDS-ring kernel (else the register-staged kernel)
    int bm, bn;     // tile
    bool eight;     // ring kernel with 8 waves (two or more rounds of tiles)
    int64_t tiles;
    int nsl, kb;    // split-K slices and 128-blocks per slice (nsl = 1: none)
    size_t part_offset, part_bytes;
};

GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k, int group)
{
    GemmPlan p{};
    p.bn = 192;
    // G = 128 reads scale pairs, which needs an even number of 128-blocks;
    // the ring kernel addresses its tensors with 32-bit offsets
    const bool small = m * k * 2 < (1LL << 32) && n * k / 2 < (1LL << 32);
    p.pipe = k % 128 == 0 && (group != 128 || (k / 128) % 2 == 0) && small;
    p.bm = (p.pipe && m <= 64) ? 64 : 128;
    p.tiles = ((n + p.bn - 1) / p.bn) * ((m + p.bm - 1) / p.bm);
    const int64_t cus = ql::cu_count();
    // 128 columns instead of 192 where 192-column tiles leave CUs idle and
    // 128 gives at least 20% more tiles in one round (13B up M=256: 144 ->
    // 216 tiles, 66 -> 54 us; fused QKV M=256: 61 -> 41 us), or, over several
    // rounds, where whole rounds x width is smaller (13B up M=1024: 3 rounds
    // of 192 against 4 of 128, 203 -> 197 us)
    if (p.pipe && p.bm == 128 && cus > 0) {
        const int64_t t128 = ((n + 127) / 128) * ((m + 127) / 128);
        const int64_t r192 = (p.tiles + cus - 1) / cus, r128 = (t128 + cus - 1) / cus;
        const bool idle = p.tiles < cus && t128 <= cus && t128 * 5 >= p.tiles * 6;
        if (idle || (p.tiles > cus && r128 * 128 < r192 * 192)) {
            p.bn = 128;
            p.tiles = t128;
        }
    }
    // 8 waves (2 x 4) for 128-row tiles: one wave per SIMD is not enough to
    // keep the matrix cores fed (13B MLP, M=256: 74 -> 65 us; fused QKV M=512
    // unchanged at ~63 us)
    p.eight = p.pipe && p.bm == 128;
    p.nsl = 1;
    p.kb = (int)(k / 128);
    if (p.pipe && cus > 0 && p.tiles < cus) {
        const int64_t nk = k / 128;
        const int64_t want = std::min<int64_t>(cus / p.tiles, nk / kGemmMinSliceBlocks);
        if (want >= 2) {
            p.kb = (int)((nk + want - 1) / want);
            p.nsl = (int)((nk + p.kb - 1) / p.kb);
        }
    }
    p.part_offset = kFixedBytes;
    p.part_bytes = p.nsl > 1 ? (size_t)p.nsl * (size_t)p.tiles * (size_t)std::min<int64_t>(m, p.bm) * (size_t)p.bn *
                                   sizeof(float)
                             : 0;
    return p;
}

size_t gemm_workspace(const GemmPlan& p) { return p.nsl > 1 ? p.part_offset + p.part_bytes : 0; }

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

template <int MT, int R, int P, bool POST, int T, int XB = 1>
void launch_decode_t(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                     const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int lg, hipStream_t st)
{
    uint32_t* cnt = p.slices > 1 ? static_cast<uint32_t*>(ws) : nullptr;
    float* part = p.slices > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                          (p.pair ? kCounterBytes : p.part_offset))
                               : nullptr;
    hipLaunchKernelGGL((w4a16_decode_kernel<MT, R, P, POST, T, XB>), dim3(p.nblk, p.slices), dim3(64 * T), p.lds_bytes,
                       st, x, qw, sc, qz, y, part, cnt, m, n, k, lg, p.ks, p.pair ? 1 : 0);
}

template <int NB, int P, bool POST>
void launch_gemv_t(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                   const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int lg, hipStream_t st)
{
    uint32_t* cnt = p.slices > 1 ? static_cast<uint32_t*>(ws) : nullptr;
    float* part = p.slices > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                          (p.pair ? kCounterBytes : p.part_offset))
                               : nullptr;
    const int pair = p.pair ? 1 : 0;
    constexpr int P0 = kGemvEarlyBlocks < P ? kGemvEarlyBlocks : P;
    if (m > 1) {
        hipLaunchKernelGGL((w4a16_gemv_kernel<NB, P, POST, kGemvMaxRows, kGemvWaves, P0>),
                           dim3(p.nblk, p.slices), dim3(64 * kGemvWaves),
                           p.lds_bytes, st, x, qw, sc, qz, y, part, cnt, m, n, k, lg, p.ks, pair);
        return;
    }
    hipLaunchKernelGGL((w4a16_gemv_kernel<NB, P, POST, 1, kGemvWaves, P0>),
                       dim3(p.nblk, p.slices), dim3(64 * kGemvWaves),
                       p.lds_bytes, st, x, qw, sc, qz, y, part, cnt, m, n, k, lg, p.ks, pair);
}

bool launch_decode(const DecodePlan& p, const uint16_t* x, const uint32_t* qw, const uint16_t* sc,
                   const uint32_t* qz, uint16_t* y, void* ws, int m, int n, int k, int lg, hipStream_t st)
{
    if (p.gemv) {
#define QL_GEMV_CASE(NB_, P_)                                                         \
    if (p.p == NB_) {                                                                 \
        if (p.post)                                                                   \
            launch_gemv_t<NB_, P_, true>(p, x, qw, sc, qz, y, ws, m, n, k, lg, st);   \
        else                                                                          \
            launch_gemv_t<NB_, P_, false>(p, x, qw, sc, qz, y, ws, m, n, k, lg, st);  \
        return true;                                                                  \
    }
        QL_GEMV_CASE(4, 4) QL_GEMV_CASE(8, 8) QL_GEMV_CASE(16, 8)
#undef QL_GEMV_CASE
        return false;
    }

#define QL_DECODE_CASE(MT_, R_, P_, T_, XB_)                                                          \
    if (p.mt == MT_ && p.r == R_ && p.p == P_ && p.t == T_) {                                         \
        if (p.post)                                                                                   \
            launch_decode_t<MT_, R_, P_, true, T_, XB_>(p, x, qw, sc, qz, y, ws, m, n, k, lg, st);    \
        else                                                                                          \
            launch_decode_t<MT_, R_, P_, false, T_, XB_>(p, x, qw, sc, qz, y, ws, m, n, k, lg, st);   \
        return true;                                                                                  \
    }
    // six-wave 16-row launches (one workgroup per CU) publish activations every second block
    QL_DECODE_CASE(16, 1, 2, 4, 1) QL_DECODE_CASE(32, 1, 2, 4, 1) QL_DECODE_CASE(16, 1, 2, 6, 2)
    QL_DECODE_CASE(32, 1, 2, 6, 1) QL_DECODE_CASE(64, 1, 2, 8, 1)
#undef QL_DECODE_CASE
    return false;
}

}  // namespace

extern "C" size_t ql_w4a16_workspace_bytes(int64_t m, int64_t n, int64_t k, int group)
{
    if (m <= 0 || n <= 0 || k <= 0 || !ql::valid_group(group) || k % group)
        return 0;
    const size_t g = gemm_workspace(gemm_plan(m, n, k, group));
    if (m > kDecodeMaxRows)
        return g;
    return std::max(g, decode_workspace(decode_plan_auto(m, n, k, group)));
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
        path = m <= kDecodeMaxRows ? QL_PATH_DECODE : QL_PATH_GEMM;
    if (path == QL_PATH_DECODE && m > kDecodeMaxRows)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: decode path needs m <= %lld (m=%lld)", who, (long long)kDecodeMaxRows,
                (long long)m);
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
        DecodePlan p = decode_plan_auto(m, n, k, group);
        if (p.slices > 1 && p.nblk > kMaxDecodeBlocks)
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: n=%lld exceeds the decode path's %d column blocks", who, (long long)n,
                    kMaxDecodeBlocks);
        if (m * k * 2 >= (1LL << 31))
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: decode activations of %lld x %lld exceed 2 GiB", who, (long long)m,
                    (long long)k);
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
            QL_FAIL(QL_ERR_UNSUPPORTED, "%s: no decode kernel for mt=%d r=%d p=%d t=%d", who, p.mt, p.r, p.p, p.t);
        return launch_status(who);
    }
    const int lg = group == 32 ? 5 : (group == 64 ? 6 : 7);
    // 128 x 192 tiles (M=512, N=12288 gives exactly one tile per CU), 64 x 192
    // for m <= 64.  4 waves (1 x 4) for launches of one round of tiles; 8
    // waves (2 x 4, each weight word dequantised twice, two waves per SIMD)
    // from two rounds on (M = 2048 fused QKV: 248 us against 260)
    using Pipe = W4PipeCfg<128, 192, 1, 3, 4>;
    using Pipe8 = W4PipeCfg<128, 192, 2, 3, 4, 8>;
    using Pipe8N = W4PipeCfg<128, 128, 2, 3, 4, 8>;   // 128 columns where 192 leave CUs idle
    using Pipe64 = W4PipeCfg<64, 192, 1, 3, 4>;
    // the same tiles with 8 waves in two k groups (two waves per SIMD, each
    // weight word still dequantised once)
    using Pipe64K = W4PipeCfg<64, 192, 1, 3, 4, 8, 2>;
    GemmPlan gp = gemm_plan(m, n, k, group);
    if (gp.pipe && !ql::lds_fits(gp.eight ? Pipe8::kLds : (gp.bm == 64 ? Pipe64::kLds : Pipe::kLds)))
        gp = GemmPlan{false, 128, 192, false, ((n + 191) / 192) * ((m + 127) / 128), 1, (int)(k / 128), 0, 0};
    const size_t need = gemm_workspace(gp);
    if (need > 0 && (!workspace || workspace_bytes < need))
        QL_FAIL(QL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !ql::aligned16(workspace))
        QL_FAIL(QL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
    if (gp.part_bytes >= ((size_t)1 << 32))
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: split-K partial sums of %zu bytes (limit 4 GiB)", who, gp.part_bytes);
    uint32_t* cnt = gp.nsl > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
    float* part = gp.nsl > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + gp.part_offset) : nullptr;
    const int64_t units = gp.tiles * gp.nsl;
    const unsigned grid = (unsigned)((units + kXcds - 1) / kXcds * kXcds);   // whole rounds over the XCDs
    if (gp.pipe) {
        if (gp.eight && gp.bn == 128)
            hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe8N>), dim3(grid), dim3(Pipe8N::NW * 64),
                               (size_t)Pipe8N::kLds, st, xw, qw, scales, qz, y, mi, ni, ki, lg, part, cnt, gp.kb,
                               gp.nsl);
        else if (gp.eight)
            hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe8>), dim3(grid), dim3(Pipe8::NW * 64), (size_t)Pipe8::kLds,
                               st, xw, qw, scales, qz, y, mi, ni, ki, lg, part, cnt, gp.kb, gp.nsl);
        else if (gp.bm == 64 && kGemmKGroups)
            hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe64K>), dim3(grid), dim3(Pipe64K::NW * 64),
                               (size_t)Pipe64K::kLds, st, xw, qw, scales, qz, y, mi, ni, ki, lg, part, cnt, gp.kb,
                               gp.nsl);
        else if (gp.bm == 64)
            hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe64>), dim3(grid), dim3(Pipe64::NW * 64),
                               (size_t)Pipe64::kLds, st, xw, qw, scales, qz, y, mi, ni, ki, lg, part, cnt, gp.kb,
                               gp.nsl);
        else
            hipLaunchKernelGGL((w4a16_gemm_pipe_kernel<Pipe>), dim3(grid), dim3(Pipe::NW * 64), (size_t)Pipe::kLds,
                               st, xw, qw, scales, qz, y, mi, ni, ki, lg, part, cnt, gp.kb, gp.nsl);
    }
    else
        hipLaunchKernelGGL((w4a16_gemm_kernel<128, 192>), dim3(grid), dim3(256), 0, st, xw, qw, scales, qz, y, mi, ni,
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

// ---------------------------------------------------------------------------
// ql_w4a16_gemm_noalloc: the same kernels with the split-K workspace in a
// file-scope device array instead of caller memory.  Each device that runs
// the library holds its own copy of `scratch` until the process ends.  Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)32 << 20;  // the fixed zero region + partial sums
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void zero_words_kernel(uint32_t* p, int count)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array; on the first call for a
// device its counter region is cleared by a small kernel on `st` (ordered
// before the caller's launch; no memset node, so the call may be captured).
int scratch_for_current_device(hipStream_t st, void** out, const char* who)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        QL_FAIL(QL_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", who, dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) {
        *out = p;
        return QL_OK;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            QL_FAIL(QL_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", who, dev,
                    hipGetErrorString(e));
        hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, st, static_cast<uint32_t*>(p),
                           (int)(kFixedBytes / sizeof(uint32_t)));
        if (int rc = launch_status(who))
            return rc;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return QL_OK;
}

}  // namespace

extern "C" int ql_w4a16_gemm_noalloc(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                                     const int32_t* qzeros, uint16_t* y, int64_t m, int64_t n, int64_t k,
                                     int group, void* stream)
{
    ql::clear_error();
    const char* who = "ql_w4a16_gemm_noalloc";
    if (int rc = check_common(qweight, scales, qzeros, n, k, group, who))
        return rc;
    if (m < 0)
        QL_FAIL(QL_ERR_SHAPE, "%s: m=%lld", who, (long long)m);
    if (m == 0 || n == 0)
        return QL_OK;
    const size_t need = ql_w4a16_workspace_bytes(m, n, k, group);
    if (need > kScratchBytes)
        QL_FAIL(QL_ERR_WORKSPACE,
                "%s: m=%lld n=%lld k=%lld needs %zu bytes of split-K scratch; this entry point holds at most %zu "
                "(use ql_w4a16_gemm with a workspace)",
                who, (long long)m, (long long)n, (long long)k, need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        if (!x || !y)
            QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
        if (int rc = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws, who))
            return rc;
    }
    return ql_w4a16_gemm_path(x, qweight, scales, qzeros, y, m, n, k, group, ws, need > 0 ? kScratchBytes : 0,
                              stream, QL_PATH_AUTO);
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
    const int64_t wblocks = n * ((k / 8 + 7) / 8);
    const unsigned blocks = (unsigned)std::min<int64_t>((wblocks + 255) / 256, 65536);
    hipLaunchKernelGGL(w4a16_dequant_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint32_t*>(qweight), scales, reinterpret_cast<const uint32_t*>(qzeros),
                       w16, q_u8, (int)n, (int)k, group);
    return launch_status(who);
}
