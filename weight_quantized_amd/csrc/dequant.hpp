// Device dequantisation of packed uint4 weights (gfx950).  The same routines
// serve the dequant export and the W4A16 kernels.  The export writes
// fp16((q - z) * s), the weights the GEMM kernels and the decode kernels at
// groups 32 and 64 contract, so its bit-exact check covers those.  The decode
// kernels at group 128 run only the first two stages (dequant_words_qz: the
// exact integers q - z) and apply s to the fp32 matrix-core result instead;
// their one-hot test checks that path bit for bit.
//
// A 32-bit word holds codes q0..q7 (code i in bits [4i, 4i+4), consecutive
// input channels).  OR-ing a nibble into the mantissa of an fp16 constant
// whose mantissa ulp equals that nibble's place value gives the constant plus
// the code, exactly, in one v_and_or_b32 for two codes 16 bits apart:
//
//   nibble at bits 0-3 of a half,  constant 1024 (0x6400, ulp 1):    1024 + q
//   nibble at bits 4-7 of a half,  constant   64 (0x5400, ulp 1/16):   64 + q
//
// Subtracting the same constant plus the zero point is exact in fp16 and
// leaves the small integer q - z; one fp16 multiply by the group scale s then
// rounds the exact product (q - z) * s once, to nearest even -- bit-identical
// to forming (q - z) * s exactly and rounding it to fp16 afterwards.
//
// Two element orders within the eight fp16 values of a word:
//   interleaved (0,4)(1,5)(2,6)(3,7): the pairs sit 16 bits apart in the word,
//     so one shift serves all four pairs (13 VALU operations per word).  The
//     activations are reordered to match (permute_x8).
//   natural (0,1)(2,3)(4,5)(6,7): v_perm_b32 copies byte i of the word into
//     bytes 0 and 2 first (16 operations per word); activations stay as they
//     are.
// Both are written stage by stage over N words -- all extractions, then all
// zero subtractions, then all scale products -- so the independent chains
// interleave instead of running back to back through one register.
// dequant_words_qz stops before the scale product: a kernel whose MFMA spans
// a single group per output channel applies the scale to the fp32 result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t u2h(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t h2u(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Per-group zero-point biases: lo = (1024 + z) in both halves, hi = (64 + z)
// in both halves, mix = (1024 + z, 64 + z) for the natural order.
struct zb_t {
    h2_t lo, hi, mix;
};
__device__ __forceinline__ zb_t make_zb(uint32_t z)
{
    const uint32_t a = 0x6400u | z, b = 0x5400u | (z << 4);
    return zb_t{u2h(a * 0x10001u), u2h(b * 0x10001u), u2h(a | (b << 16))};
}
// the fp16 scale in both halves
__device__ __forceinline__ h2_t scale2(uint32_t s16) { return u2h(s16 * 0x10001u); }

// (w & mask) | magic in one VALU instruction.  The compiler otherwise splits
// it into an AND and an OR.  VOP3 may read one scalar register: the mask sits
// in an SGPR, the magic constant in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// N words -> N x 8 fp16 values q - z (exact small integers) in the order
// (0,4)(1,5)(2,6)(3,7), as four pairs per word.
template <int N>
__device__ __forceinline__ void dequant_words_qz(const uint32_t (&w)[N], const zb_t (&zb)[N], h2_t (&d)[N][4])
{
    constexpr uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u, kMLo = 0x64006400u, kMHi = 0x54005400u;
    uint32_t e[N][4];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const uint32_t w8 = w[j] >> 8;
        e[j][0] = and_or(w[j], kLo, kMLo);   // codes 0, 4
        e[j][1] = and_or(w[j], kHi, kMHi);   // codes 1, 5
        e[j][2] = and_or(w8, kLo, kMLo);     // codes 2, 6
        e[j][3] = and_or(w8, kHi, kMHi);     // codes 3, 7
    }
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[j][i] = u2h(e[j][i]) - ((i & 1) ? zb[j].hi : zb[j].lo);
}

// N words -> N x 8 fp16 weights in the order (0,4)(1,5)(2,6)(3,7).
template <int N>
__device__ __forceinline__ void dequant_words(const uint32_t (&w)[N], const zb_t (&zb)[N], const h2_t (&s2)[N],
                                              h8_t (&out)[N])
{
    h2_t d[N][4];
    dequant_words_qz<N>(w, zb, d);
#pragma unroll
    for (int j = 0; j < N; ++j)
        out[j] = __builtin_bit_cast(h8_t, make_uint4(h2u(d[j][0] * s2[j]), h2u(d[j][1] * s2[j]),
                                                     h2u(d[j][2] * s2[j]), h2u(d[j][3] * s2[j])));
}

// N words -> N x 8 fp16 weights in natural order.
template <int N>
__device__ __forceinline__ void dequant_words_natural(const uint32_t (&w)[N], const zb_t (&zb)[N],
                                                      const h2_t (&s2)[N], h8_t (&out)[N])
{
    constexpr uint32_t kMask = 0x00F0000Fu, kMagic = 0x54006400u;
    uint32_t e[N][4];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // selector bytes: [byte i, zero, byte i, zero]
            const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)i << 16) | (0x0Cu << 24);
            e[j][i] = and_or(__builtin_amdgcn_perm(w[j], w[j], sel), kMask, kMagic);
        }
    h2_t d[N][4];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[j][i] = u2h(e[j][i]) - zb[j].mix;
#pragma unroll
    for (int j = 0; j < N; ++j)
        out[j] = __builtin_bit_cast(h8_t, make_uint4(h2u(d[j][0] * s2[j]), h2u(d[j][1] * s2[j]),
                                                     h2u(d[j][2] * s2[j]), h2u(d[j][3] * s2[j])));
}

// Eight consecutive fp16 activations (as four 32-bit pairs) -> the order
// (0,4)(1,5)(2,6)(3,7) that matches dequant_words: one v_perm_b32 per output
// dword, selecting two bytes from each of two input dwords.  With the
// selectors sel_lo = kPermLo, sel_hi = kPermHi it reorders; with kPermZero
// (selector byte 0x0C reads as 0x00) it writes zeros instead, so a masked
// chunk costs no extra instruction.
constexpr uint32_t kPermLo = 0x05040100u;     // [a.b0, a.b1, b.b0, b.b1] of perm(b, a)
constexpr uint32_t kPermHi = 0x07060302u;     // [a.b2, a.b3, b.b2, b.b3]
constexpr uint32_t kPermZero = 0x0C0C0C0Cu;
__device__ __forceinline__ uint4 permute_x8_sel(uint4 v, uint32_t sel_lo, uint32_t sel_hi)
{
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, sel_lo), __builtin_amdgcn_perm(v.z, v.x, sel_hi),
                      __builtin_amdgcn_perm(v.w, v.y, sel_lo), __builtin_amdgcn_perm(v.w, v.y, sel_hi));
}
__device__ __forceinline__ uint4 permute_x8(uint4 v) { return permute_x8_sel(v, kPermLo, kPermHi); }

// Zero point of group g of one row: nibble g%8 of word g/8.
__device__ __forceinline__ uint32_t zero_of(const uint32_t* qz_row, int g)
{
    return (qz_row[g >> 3] >> (4 * (g & 7))) & 0xFu;
}

}  // namespace ql
