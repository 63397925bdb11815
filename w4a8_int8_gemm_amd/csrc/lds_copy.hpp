// Device helpers of the GEMM kernels: direct-to-LDS copies, explicit waits,
// buffer resources and an LDS-only barrier (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace w4a8 {

// Swap lanes 32-63 of x with lanes 0-31 of y (v_permlane32_swap): lane l < 32
// keeps x and receives y of lane l + 32 in y; lane l + 32 receives x of lane l
// in x and keeps y.
__device__ __forceinline__ void lane_half_swap(uint32_t &x, uint32_t &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
}

// Workgroup barrier that orders LDS accesses only: global loads stay in
// flight across it (a full __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS copies: each lane's bytes from global memory land at
// M0 + size * lane.  Issued through asm so that the only waits on them are
// the kernel's own (vmcnt before the barrier that publishes a stage); the
// "memory" clobber keeps other memory accesses from moving across them.  One
// wait state separates the SALU write of M0 from the load that reads it (a
// gfx9 hazard).  M0 is not restored: nothing else in these kernels uses it
// (the compiler cannot be told that asm writes M0, so a CPU test checks the
// kernels' assembly for any other M0 access).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}
__device__ __forceinline__ void copy4_to_lds(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "memory");
}

// s_waitcnt that waits for the vector-memory counter only (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maximum).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Buffer resource of a raw byte range [base, base + bytes): loads at offsets
// past `bytes` return zeros instead of touching memory.
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;                                  // gfx9 raw buffer: 32-bit data format
    return r;
}

// M0 = the LDS address the next direct-to-LDS buffer loads write at.
__device__ __forceinline__ void set_m0(uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(lds) : "memory");
}

// 16 bytes per lane from a buffer resource into LDS at M0 + OFF + 16 * lane,
// from byte offset voff + OFF (+ soff) of the resource.  The immediate OFF
// adds to both addresses and takes part in the range check: lanes whose
// voff + OFF lies past the resource's size read zeros.  M0 must hold the
// LDS base (set_m0); nothing else in these kernels touches M0.
template <int OFF>
__device__ __forceinline__ void copy16_buf_to_lds(v4i rsrc, uint32_t voff, uint32_t soff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF)
                 : "memory");
}

}  // namespace w4a8
