// Symmetric quantization rule shared by every kernel of the library.
//
// The four-step pipeline of the Apple-silicon essay ("Apple Silicon의 AI
// 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계") derives
// a scale from a min/max reduction and maps values to INT8 with it.  The
// pages give no formula; the rule implemented here is
//     s = fl32(amax / qmax),  q = clamp(round_half_away(fl32(x / s)), -qmax, qmax)
// with qmax = 127 (int8) or 7 (int4) and true IEEE fp32 division.
//
// Two ways to reach the same code:
//  * quant_code_div: the rule as written (one IEEE division per element);
//  * quant_code_fast: one fma with r = fl32(1/s) plus a guard.  The fma
//    result v = fl32(|x| r + 1/2) differs from |fl32(x/s)| + 1/2 by less than
//    2^-15 whenever |x/s| <= 128 (r carries one rounding, the fma one more,
//    the division one), so floor(v) equals round_half_away(fl32(x/s)) unless
//    v lies within 2^-15 of an integer.  The guard flags every v within 2^-14
//    of an integer; those elements must be recomputed with quant_code_div.
//
// This header is also compiled for the host by the CPU test suite, which
// checks the fast path plus guard against the division rule on every fp16
// input for many scales.
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define W4A8_HD __host__ __device__ __forceinline__
#else
#include <math.h>
#define W4A8_HD static inline
#endif

namespace w4a8 {

W4A8_HD float quant_scale(float amax, float qmax) { return amax / qmax; }

// The rule as written.  s == 0 only for an all-zero slice, whose codes are 0.
W4A8_HD int quant_code_div(float x, float s, float qmax)
{
    if (s == 0.0f)
        return 0;
    float t = x / s;
    float r = roundf(t);                       // halves go away from zero
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int)r;
}

// Guard width: v within this distance of an integer goes to the slow path.
#define W4A8_QUANT_GUARD 0x1p-14f

// Fast path.  `r` is fl32(1/s) for s != 0.  Sets `slow` (never clears it)
// when the element must be recomputed with quant_code_div.
W4A8_HD int quant_code_fast(float x, float r, float qmax, bool &slow)
{
    float v = fmaf(fabsf(x), r, 0.5f);
    float f = floorf(v);
    float d = v - f;                           // exact: v and f share a binade
    slow |= fabsf(d - 0.5f) > 0.5f - W4A8_QUANT_GUARD;
    f = fminf(f, qmax);
    return (int)copysignf(f, x);
}

}  // namespace w4a8
