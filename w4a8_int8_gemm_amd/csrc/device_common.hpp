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

// Two fp32 values to two fp16 (a in the low half), each rounded to nearest
// even as f2h does, in one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    asm("" : "+v"(a), "+v"(b));
    const h2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Four int codes in [-127, 127] to four bytes, element 0 in the low byte.
__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)d << 24);
}

// Reductions over groups of `width` consecutive lanes (2, 4, 8, 16 or 64)
// with DPP lane moves.  Within a row of 16 lanes: swap neighbours, then
// pairs (quad permutes), then mirror half rows and rows -- after each move
// every lane of a group holds the group's value, and its partner lies in the
// sibling group.  Across the four rows of a wave: row broadcasts carry row 0
// into row 1 and row 2 into row 3, then the lower half into the upper; lane
// 63 ends with the total, which is read into every lane.  Lanes that a move
// does not reach take 0, the identity of both max (of unsigned values) and +.
#define W4A8_DPP(x, ctrl, rows) __builtin_amdgcn_update_dpp(0, (x), (ctrl), (rows), 0xf, false)

template <int width, typename T, typename Op>
__device__ __forceinline__ T lane_reduce(T v, Op op)
{
    static_assert(width == 2 || width == 4 || width == 8 || width == 16 || width == 64,
                  "reduction width");
    v = op(v, (T)W4A8_DPP((int)v, 0xb1, 0xf));          // quad_perm [1,0,3,2]
    if constexpr (width >= 4)
        v = op(v, (T)W4A8_DPP((int)v, 0x4e, 0xf));      // quad_perm [2,3,0,1]
    if constexpr (width >= 8)
        v = op(v, (T)W4A8_DPP((int)v, 0x141, 0xf));     // row_half_mirror
    if constexpr (width >= 16)
        v = op(v, (T)W4A8_DPP((int)v, 0x140, 0xf));     // row_mirror
    if constexpr (width == 64) {
        v = op(v, (T)W4A8_DPP((int)v, 0x142, 0xa));     // row_bcast:15 into rows 1, 3
        v = op(v, (T)W4A8_DPP((int)v, 0x143, 0xc));     // row_bcast:31 into rows 2, 3
        v = (T)__builtin_amdgcn_readlane((int)v, 63);
    }
    return v;
}

template <int width>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v)
{
    return lane_reduce<width>(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}

template <int width>
__device__ __forceinline__ int group_sum_i32(int v)
{
    return lane_reduce<width>(v, [](int a, int b) { return a + b; });
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

// fl32(x r) for the fp16 x in the low (HI false) or high half of w, in one
// v_fma_mix_f32: the fp16 converts exactly and the addend is +0, so the
// result is the rounded product (a zero product comes out as +0).
template <bool HI>
__device__ __forceinline__ float h2f_times(uint32_t w, float r)
{
    float t;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(t) : "v"(w), "v"(r));
    else
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(t) : "v"(w), "v"(r));
    return t;
}

// Bytes 0 of the bit patterns of a, b, c, d as one dword (a lowest).
__device__ __forceinline__ uint32_t low_bytes4(float a, float b, float c, float d)
{
    const uint32_t ab = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x04000c0cu);
    return ab | cd;
}

// Quantize the eight fp16 values of a chunk with scale s (r = fl32(1/s)),
// in two parts (quant_chunk8 runs the first, and the second only when the
// guard trips):
//  * quant_chunk8_fast: t = fl32(x r); m = t + 1.5 * 2^23 rounds t to the
//    nearest integer (ties to even, |t| < 2^22) and holds it, two's
//    complement, in its low mantissa bits, so byte 0 of m is the code and
//    m - 1.5 * 2^23 (exact) is rint(t); the largest distance |t - rint(t)|
//    of the eight is folded into `far` for the guard;
//  * quant_chunk8_div: the division rule's codes for all eight, from the
//    corrected quotient q = fl32(x / s) (quant_div_corrected: no division
//    instruction); q + 1.5 * 2^23 holds rint(q) in byte 0 as above, which is
//    round_half_away(q) unless q is exactly a half-integer -- a chunk holding
//    such a tie takes quant_code_corrected (roundf) for all eight.
// A chunk whose distance trips the guard takes the division rule whole; a
// zero scale (all-zero slice) gives zero codes.
__device__ __forceinline__ uint2 quant_chunk8_fast(uint4 v, float r, float &far)
{
    constexpr float kRound = 0x1.8p23f;
    const float t[8] = {h2f_times<false>(v.x, r), h2f_times<true>(v.x, r),
                        h2f_times<false>(v.y, r), h2f_times<true>(v.y, r),
                        h2f_times<false>(v.z, r), h2f_times<true>(v.z, r),
                        h2f_times<false>(v.w, r), h2f_times<true>(v.w, r)};
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m[i] = t[i] + kRound;
        far = fmaxf(far, fabsf(t[i] - (m[i] - kRound)));
    }
    return make_uint2(low_bytes4(m[0], m[1], m[2], m[3]), low_bytes4(m[4], m[5], m[6], m[7]));
}

__device__ __forceinline__ uint2 quant_chunk8_div(uint4 v, float s, float r, float qmax)
{
    constexpr float kRound = 0x1.8p23f;
    const float x[8] = {lo_h2f(v.x), hi_h2f(v.x), lo_h2f(v.y), hi_h2f(v.y),
                        lo_h2f(v.z), hi_h2f(v.z), lo_h2f(v.w), hi_h2f(v.w)};
    float m[8];
    float tie = 0.0f;                 // largest |q - rint(q)|: 1/2 only for an exact tie
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = quant_div_corrected(x[i], s, r);
        m[i] = q + kRound;
        tie = fmaxf(tie, fabsf(q - (m[i] - kRound)));
    }
    if (__builtin_expect(tie == 0.5f, 0)) {
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = quant_code_corrected(x[i], s, r, qmax);
        return make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
    }
    return make_uint2(low_bytes4(m[0], m[1], m[2], m[3]), low_bytes4(m[4], m[5], m[6], m[7]));
}

// Both parts for one chunk, the guard tested per chunk.
__device__ __forceinline__ uint2 quant_chunk8(uint4 v, float s, float r, float qmax)
{
    if (s == 0.0f)
        return make_uint2(0u, 0u);
    float far = 0.0f;
    const uint2 c = quant_chunk8_fast(v, r, far);
    if (__builtin_expect(quant_fast_slow(far), 0))
        return quant_chunk8_div(v, s, r, qmax);
    return c;
}

// Per-channel rescale of one int32 sum; the same operation order everywhere
// (GEMM epilogue and matrix-vector kernel), so both give identical fp16 bits.
__device__ __forceinline__ float rescale_pc(int c, float sa, float sw)
{
    return ((float)c * sa) * sw;
}

}  // namespace w4a8
