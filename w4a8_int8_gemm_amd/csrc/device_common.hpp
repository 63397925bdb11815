// Device-side helpers shared by the library's HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quant_rule.h"

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte load that is not expected to be reused (streamed once).
__device__ __forceinline__ uint4 load_nt(const uint4 *p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// fp16 bits <-> fp32.  Widening is exact; narrowing rounds the fp32 value to
// nearest even (v_cvt_f16_f32).  The empty asm keeps the instruction selector
// from fusing a preceding fp32 multiply into the conversion (v_fma_mixlo_f16
// rounds once, straight to fp16), so every kernel rounds the same fp32 value
// the same way.
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f)
{
    asm("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two fp16 values (low, high half of a dword) to fp32.
__device__ __forceinline__ float lo_h2f(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float hi_h2f(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}

// Four int codes in [-127, 127] to four bytes, element 0 in the low byte.
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)d << 24);
}

// Butterfly max over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 1; off < width; off <<= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

template <int width>
__device__ __forceinline__ int group_sum_i32(int v)
{
#pragma unroll
    for (int off = 1; off < width; off <<= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// max(|h|) of the eight fp16 values in a 16-byte chunk, as fp16 bits.  For
// non-negative fp16 the bit patterns order like the values, so the maximum
// is taken on the integers after clearing the sign bits.
__device__ __forceinline__ uint32_t absmax_bits8(uint4 v)
{
    uint32_t a = v.x & 0x7fff7fffu, b = v.y & 0x7fff7fffu, c = v.z & 0x7fff7fffu,
             d = v.w & 0x7fff7fffu;
    uint32_t m0 = max(a & 0xffffu, a >> 16), m1 = max(b & 0xffffu, b >> 16);
    uint32_t m2 = max(c & 0xffffu, c >> 16), m3 = max(d & 0xffffu, d >> 16);
    return max(max(m0, m1), max(m2, m3));
}

// Quantize the eight fp16 values of a chunk with scale s (r = fl32(1/s)).
// Fast path for all eight; any guarded element sends the whole chunk through
// the division rule.  Returns the eight codes as two dwords.
__device__ __forceinline__ uint2 quant_chunk8(uint4 v, float s, float r, float qmax)
{
    if (s == 0.0f)
        return make_uint2(0u, 0u);
    float x0 = lo_h2f(v.x), x1 = hi_h2f(v.x), x2 = lo_h2f(v.y), x3 = hi_h2f(v.y);
    float x4 = lo_h2f(v.z), x5 = hi_h2f(v.z), x6 = lo_h2f(v.w), x7 = hi_h2f(v.w);
    bool slow = false;
    int q0 = quant_code_fast(x0, r, qmax, slow), q1 = quant_code_fast(x1, r, qmax, slow);
    int q2 = quant_code_fast(x2, r, qmax, slow), q3 = quant_code_fast(x3, r, qmax, slow);
    int q4 = quant_code_fast(x4, r, qmax, slow), q5 = quant_code_fast(x5, r, qmax, slow);
    int q6 = quant_code_fast(x6, r, qmax, slow), q7 = quant_code_fast(x7, r, qmax, slow);
    if (__builtin_expect(slow, 0)) {
        q0 = quant_code_div(x0, s, qmax); q1 = quant_code_div(x1, s, qmax);
        q2 = quant_code_div(x2, s, qmax); q3 = quant_code_div(x3, s, qmax);
        q4 = quant_code_div(x4, s, qmax); q5 = quant_code_div(x5, s, qmax);
        q6 = quant_code_div(x6, s, qmax); q7 = quant_code_div(x7, s, qmax);
    }
    return make_uint2(pack_i8x4(q0, q1, q2, q3), pack_i8x4(q4, q5, q6, q7));
}

// Per-channel rescale of one int32 sum; the same operation order everywhere
// (GEMM epilogue and matrix-vector kernel), so both give identical fp16 bits.
__device__ __forceinline__ float rescale_pc(int c, float sa, float sw)
{
    return ((float)c * sa) * sw;
}

}  // namespace w4a8
