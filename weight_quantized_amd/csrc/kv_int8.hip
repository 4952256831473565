// KV-cache INT8 group quantisation for gfx950 and its C-ABI entry points
// (FastLLM architecture page, section 5.2: the KV cache quantised between FP16
// and INT8 in groups of 128, dequantised when read).
//
//   kv_quant_kernel   -- fp16 groups of G -> int8 codes + one fp32 scale each
//   kv_dequant_kernel -- int8 codes + scales -> fp16
//
// Both stream HBM once: a quantised group is G fp16 in, G int8 + 4 bytes out.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ql_common.hpp"

namespace {

__device__ __forceinline__ float h2f(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

// One thread per 16-byte chunk (8 values); the G / 8 threads of a group are
// consecutive lanes of one wave and reduce max|x| with butterfly shuffles.
// scale = max|x| / 127 and code = clamp(rint(x / scale), -127, 127), both
// correctly rounded fp32 divisions: q0 = x * RN(1/scale) is within 1.5 ulp of
// fp32(x / scale) (|q0| <= 127, an ulp at most 2^-17), so both round to the same
// integer unless q0 lies within 2^-15 of a half-integer; only those divide.
template <int G>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ x, int8_t* __restrict__ q,
                                                       float* __restrict__ scale, int64_t chunks)
{
    constexpr int TPG = G / 8;                         // threads per group
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool ok = c < chunks;
    const uint4 v = ok ? reinterpret_cast<const uint4*>(x)[c] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = h2f(w[e] & 0xFFFFu);
        f[2 * e + 1] = h2f(w[e] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
    for (int d = 1; d < TPG; d <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, d, TPG));
    const float sc = __fdiv_rn(amax, 127.0f);
    if (!ok)
        return;
    if ((threadIdx.x & (TPG - 1)) == 0)
        scale[c / TPG] = sc;
    const float rcp = sc > 0.0f ? __fdiv_rn(1.0f, sc) : 0.0f;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t code = 0u;
        if (sc > 0.0f) {
            const float q0 = f[e] * rcp;
            float qr = rintf(q0);
            if (__builtin_expect(fabsf(q0 - (floorf(q0) + 0.5f)) <= 0x1p-15f, 0))
                qr = rintf(__fdiv_rn(f[e], sc));
            code = (uint32_t)(int)fminf(fmaxf(qr, -127.0f), 127.0f) & 0xFFu;
        }
        packed[e >> 2] |= code << (8 * (e & 3));
    }
    reinterpret_cast<uint2*>(q)[c] = make_uint2(packed[0], packed[1]);
}

// One thread per 16 codes; out = fp16(fp32(q * scale)).
template <int G>
__global__ __launch_bounds__(256) void kv_dequant_kernel(const int8_t* __restrict__ q, const float* __restrict__ scale,
                                                         uint16_t* __restrict__ out, int64_t chunks)
{
    constexpr int TPG = G / 16;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks)
        return;
    const uint4 v = reinterpret_cast<const uint4*>(q)[c];
    const float sc = scale[c / TPG];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int8_t lo = (int8_t)(w[e >> 1] >> (16 * (e & 1)));
        const int8_t hi = (int8_t)(w[e >> 1] >> (16 * (e & 1) + 8));
        const float a = (float)lo * sc, b = (float)hi * sc;
        o[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
    }
    uint4* po = reinterpret_cast<uint4*>(out) + 2 * c;
    po[0] = make_uint4(o[0], o[1], o[2], o[3]);
    po[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

int check_kv(const void* a, const void* b, const void* c, int64_t groups, int group, const char* who)
{
    if (!ql::valid_group(group))
        QL_FAIL(QL_ERR_GROUP, "%s: group %d not in {32, 64, 128}", who, group);
    if (groups < 0)
        QL_FAIL(QL_ERR_SHAPE, "%s: groups=%lld", who, (long long)groups);
    if (groups > (1LL << 40) / group)
        QL_FAIL(QL_ERR_UNSUPPORTED, "%s: groups=%lld too many", who, (long long)groups);
    if (groups == 0)
        return QL_OK;
    if (!a || !b || !c)
        QL_FAIL(QL_ERR_NULL, "%s: null pointer", who);
    if (!ql::aligned16(a) || !ql::aligned16(b) || !ql::aligned16(c))
        QL_FAIL(QL_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", who);
    return QL_OK;
}

int kv_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        QL_FAIL(QL_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return QL_OK;
}

}  // namespace

extern "C" int ql_kv_quant_int8(const uint16_t* x, int8_t* q, float* scale, int64_t groups, int group, void* stream)
{
    ql::clear_error();
    const char* who = "ql_kv_quant_int8";
    if (int rc = check_kv(x, q, scale, groups, group, who))
        return rc;
    if (groups == 0)
        return QL_OK;
    const int64_t chunks = groups * (group / 8);
    const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (group == 32)
        hipLaunchKernelGGL(kv_quant_kernel<32>, grid, block, 0, st, x, q, scale, chunks);
    else if (group == 64)
        hipLaunchKernelGGL(kv_quant_kernel<64>, grid, block, 0, st, x, q, scale, chunks);
    else
        hipLaunchKernelGGL(kv_quant_kernel<128>, grid, block, 0, st, x, q, scale, chunks);
    return kv_status(who);
}

extern "C" int ql_kv_dequant_int8(const int8_t* q, const float* scale, uint16_t* out, int64_t groups, int group,
                                  void* stream)
{
    ql::clear_error();
    const char* who = "ql_kv_dequant_int8";
    if (int rc = check_kv(q, scale, out, groups, group, who))
        return rc;
    if (groups == 0)
        return QL_OK;
    const int64_t chunks = groups * (group / 16);
    const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (group == 32)
        hipLaunchKernelGGL(kv_dequant_kernel<32>, grid, block, 0, st, q, scale, out, chunks);
    else if (group == 64)
        hipLaunchKernelGGL(kv_dequant_kernel<64>, grid, block, 0, st, q, scale, out, chunks);
    else
        hipLaunchKernelGGL(kv_dequant_kernel<128>, grid, block, 0, st, q, scale, out, chunks);
    return kv_status(who);
}
