// Direct global->LDS loads and the LDS-ring handshake shared by the pipelined
// GEMM kernels (gfx950).
//
// A direct load moves each lane's 16 bytes from global memory into LDS at
// M0 + 16 * lane, so one wave instruction fills 1 KiB of LDS contiguously
// without passing through registers.  The compiler does not track which LDS
// bytes such a load writes and would wait for every outstanding load before
// any LDS read; the loads and the waits are therefore written here in inline
// assembly and each kernel counts its own outstanding loads.
//
// LDS rows are XOR-swizzled in 16-byte chunks: logical chunk c of row r is
// stored at chunk c ^ f(r).  The functions below were chosen by measurement
// (the LDS bank-conflict counter, SQ_LDS_BANK_CONFLICT, on gfx950) for the
// fragment reads the kernels make -- lane (q, r16) of a 64-lane ds_read_b128
// reading row 16 i + r16 -- and give zero conflicts there, where the plain
// layouts give 2- to 8-way conflicts.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace ql {

// one direct load: each lane's 16 bytes at `src` -> LDS `lds_base` + 16 * lane
// (lds_base must be wave-uniform)
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base)
{
    asm volatile("global_load_lds_dwordx4 %1, off" : : "{m0}"(lds_base), "v"(src) : "memory");
}

// 4-byte direct load: each lane's dword at `src` -> LDS `lds_base` + 4 * lane
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base)
{
    asm volatile("global_load_lds_dword %1, off" : : "{m0}"(lds_base), "v"(src) : "memory");
}

// The same two loads addressed as a wave-uniform 64-bit base (scalar
// registers) plus a 32-bit per-lane byte offset (the instructions' saddr
// form), so a lane keeps one register per load instead of a 64-bit address.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base)
{
    asm volatile("global_load_lds_dwordx4 %1, %2" : : "{m0}"(lds_base), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t lds_base)
{
    asm volatile("global_load_lds_dword %1, %2" : : "{m0}"(lds_base), "v"(off), "s"(base) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are pending
// (they complete in issue order) and its LDS reads have returned, then
// synchronise the workgroup.  Also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void stage_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

//   64-byte rows (4 chunks), lane quarter q reads chunk q
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 2; }
// Rows read by 32-row MFMA fragments (lane half h reads chunk 2j + h of row
// l % 32), swizzles measured free of bank conflicts on gfx950:
//   64-byte rows (4 chunks); swz64 above conflicts 2-way here
__device__ __forceinline__ int swz64x32(int r) { return (r >> 3) & 3; }
//   128-byte rows (8 chunks): swz128 below, which also serves 16-row reads
//
// 128-byte rows (8 chunks), lane quarter q reads chunk 4j + q
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }
//   256-byte rows (16 chunks), lane quarter q reads chunk 4q + s: the linear
//   map with bit images 1 -> 4, 2 -> 2, 4 -> 8, 8 -> 3 on the low four row bits
__device__ __forceinline__ int swz256(int r)
{
    return (((r & 1) << 2) | (r & 2) | ((r & 4) << 1)) ^ (((r >> 3) & 1) * 3);
}

// Host: whether the current device grants `bytes` of LDS to one workgroup
// (gfx950: 160 KiB); queried once per device.
// Host: compute units of the current device, queried once per device (0 if
// the query fails).
inline int cu_count()
{
    static std::atomic<int> cus[64];   // compute units + 1; 0 = not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        v = n + 1;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

inline bool lds_fits(int bytes)
{
    static std::atomic<int> cap[64];   // LDS bytes per workgroup + 1; 0 = not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return false;
    int v = cap[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            lds = 0;
        v = lds + 1;
        cap[dev].store(v, std::memory_order_relaxed);
    }
    return bytes <= v - 1;
}

}  // namespace ql
