// Device dequantisation of packed uint4 weights (gfx950).  One routine is
// shared by the dequant export and both W4A16 GEMM paths, so the bit-exact
// check of the export covers the values the GEMMs contract.
//
// A 32-bit word holds codes q0..q7 (code i in bits [4i, 4i+4), consecutive
// input channels).  Masking two nibbles that sit 16 bits apart and OR-ing in
// 0x6400 (fp16 1024.0, whose mantissa ulp is 1) gives the fp16 pair
// (1024 + qi, 1024 + q(i+4)) in one VALU instruction.  Subtracting
// (1024 + z) is exact in fp16 and leaves the small integer q - z; one fp16
// multiply by the group scale s then rounds the exact product (q - z) * s
// once, to nearest even.  This is bit-identical to computing (q - z) * s
// exactly and rounding it to fp16 afterwards.
//
// Output element order within the 8 lanes of a word: (0,4) (1,5) (2,6) (3,7).
// Contractions take the activation chunk in the same order (permute_x8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t u2h(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t h2u(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// (1024 + z) in both halves, z = zero point of the group.
__device__ __forceinline__ h2_t zero_bias(uint32_t z) { return u2h((0x6400u | z) * 0x10001u); }
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

// Eight codes of one word -> eight fp16 weights in the order (0,4)(1,5)(2,6)(3,7).
__device__ __forceinline__ void dequant_word(uint32_t w, h2_t zb, h2_t s2, h2_t out[4])
{
    constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
    out[0] = (u2h(and_or(w, kMask, kMagic)) - zb) * s2;
    out[1] = (u2h(and_or(w >> 4, kMask, kMagic)) - zb) * s2;
    out[2] = (u2h(and_or(w >> 8, kMask, kMagic)) - zb) * s2;
    out[3] = (u2h(and_or(w >> 12, kMask, kMagic)) - zb) * s2;
}

// dequant_word packed as one 8-half MFMA operand
__device__ __forceinline__ h8_t dequant_word8(uint32_t w, h2_t zb, h2_t s2)
{
    h2_t o[4];
    dequant_word(w, zb, s2, o);
    return __builtin_bit_cast(h8_t, make_uint4(h2u(o[0]), h2u(o[1]), h2u(o[2]), h2u(o[3])));
}

// dequant_word8 over the eight words of a 256-k decode block (words 0-3 in
// group a, 4-7 in group b), written stage by stage -- all extractions, then
// all zero subtractions, then all scale products -- so the 32 independent
// chains interleave instead of running back to back through one register.
__device__ __forceinline__ void dequant_block8(const uint32_t (&w)[8], const h2_t (&zb)[2], const h2_t (&s2)[2],
                                               h8_t (&out)[8])
{
    constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
    uint32_t e[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            e[j][i] = and_or(w[j] >> (4 * i), kMask, kMagic);
    h2_t d[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[j][i] = u2h(e[j][i]) - zb[j >> 2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        out[j] = __builtin_bit_cast(h8_t, make_uint4(h2u(d[j][0] * s2[j >> 2]), h2u(d[j][1] * s2[j >> 2]),
                                                     h2u(d[j][2] * s2[j >> 2]), h2u(d[j][3] * s2[j >> 2])));
}

// Same values as dequant_word8 in natural element order (0,1)(2,3)(4,5)(6,7):
// with w4 = w >> 4, v_perm_b32 places byte i of w (low nibble n_2i) in byte 0
// and byte i of w4 (low nibble n_2i+1) in byte 2, then the same mask-and-bias
// and the same two packed operations as above.  Two more instructions per word
// than dequant_word8, but the activations need no reordering.
__device__ __forceinline__ h8_t dequant_word8_natural(uint32_t w, h2_t zb, h2_t s2)
{
    constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
    const uint32_t w4 = w >> 4;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // selector bytes: [i of w, zero, i of w4, zero]; w4 is bytes 4..7 of the pair
        const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
        const uint32_t p = __builtin_amdgcn_perm(w4, w, sel);
        o[i] = h2u((u2h(and_or(p, kMask, kMagic)) - zb) * s2);
    }
    return __builtin_bit_cast(h8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// dequant_word8_natural over N words (each with its own zero bias and
// scale), written stage by stage so the independent chains interleave.
template <int N>
__device__ __forceinline__ void dequant_words_natural(const uint32_t (&w)[N], const h2_t (&zb)[N],
                                                      const h2_t (&s2)[N], h8_t (&out)[N])
{
    constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
    uint32_t e[N][4];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const uint32_t w4 = w[j] >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
            e[j][i] = and_or(__builtin_amdgcn_perm(w4, w[j], sel), kMask, kMagic);
        }
    }
    h2_t d[N][4];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[j][i] = u2h(e[j][i]) - zb[j];
#pragma unroll
    for (int j = 0; j < N; ++j)
        out[j] = __builtin_bit_cast(h8_t, make_uint4(h2u(d[j][0] * s2[j]), h2u(d[j][1] * s2[j]),
                                                     h2u(d[j][2] * s2[j]), h2u(d[j][3] * s2[j])));
}

// Eight consecutive fp16 activations (as four 32-bit pairs) -> the order
// (0,4)(1,5)(2,6)(3,7) that matches dequant_word.
__device__ __forceinline__ uint4 permute_x8(uint4 v)
{
    uint4 p;
    p.x = (v.x & 0xFFFFu) | (v.z << 16);
    p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p.z = (v.y & 0xFFFFu) | (v.w << 16);
    p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return p;
}

// Zero point of group g of one row: nibble g%8 of word g/8.
__device__ __forceinline__ uint32_t zero_of(const uint32_t* qz_row, int g)
{
    return (qz_row[g >> 3] >> (4 * (g & 7))) & 0xFu;
}

}  // namespace ql
