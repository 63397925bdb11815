// Symmetric quantization rule shared by every kernel of the library.
//
// The four-step pipeline of the Apple-silicon essay ("Apple Silicon의 AI
// 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계") derives
// a scale from a min/max reduction and maps values to INT8 with it.  The
// pages give no formula; the rule implemented here is
//     s = fl32(amax / qmax),  q = clamp(round_half_away(fl32(x / s)), -qmax, qmax)
// with qmax = 127 (int8) or 7 (int4) and true IEEE fp32 division.
//
// Three ways to reach the same code:
//  * quant_code_div: the rule as written (one IEEE division per element);
//  * quant_code_corrected (below): the same quotient from the reciprocal and
//    one fma correction, exact on the kernels' whole input domain;
//  * quant_code_fast: t = fl32(x r) with r = fl32(1/s), code rint(t), plus a
//    guard.  t differs from x/s by at most |x/s| 2^-23 (r and the product
//    carry one rounding each), which is below 1.6e-5 for |x/s| <= 128, so
//    rint(t) equals round_half_away(fl32(x/s)) unless x/s lies within that
//    distance of a half-integer.  The guard flags every t whose distance to
//    its nearest integer exceeds 1/2 - 2^-14 (exact ties included, where rint
//    and round_half_away differ); those elements take quant_code_div (the
//    kernels: quant_code_corrected, the same codes).  The
//    clamp is never active on this path: with |x| <= amax (s is derived from
//    the slice's own amax), |t| <= qmax (1 + 2^-22) < qmax + 1/2 - 2^-14.
//    The test is split so a kernel can take the maximum distance over
//    several elements and compare once.
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

// s = fl32(amax / qmax) without a division instruction: with c = fl32(1/qmax)
// and s0 = fl32(amax c), one correction step fl32(s0 + (amax - s0 qmax) c)
// (the residual exact by one fma) gives the quotient; the host test suite
// checks it bit for bit against the division for every fp16 amax, infinity
// included, at qmax = 127 and 7 -- the only values the kernels use.  An
// infinite amax keeps the division's infinite scale (the correction would
// turn it into NaN).
W4A8_HD float quant_scale(float amax, float qmax)
{
    const float c = 1.0f / qmax;
    const float s0 = amax * c;
    const float s = fmaf(fmaf(-s0, qmax, amax), c, s0);
    return s0 == INFINITY ? s0 : s;
}

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

// The quotient fl32(x / s) without a division instruction, for the guarded
// elements: with r = fl32(1/s) (correctly rounded) and t = fl32(x r), the
// residual e = x - t s is computed exactly by one fma, and fl32(t + e r) is
// the correctly rounded quotient (one correction step of the reciprocal
// method).  The CPU test suite checks that it equals x / s bit for bit for
// every fp16 x with |x| <= amax and every fp16 amax, s = fl32(amax / qmax),
// qmax = 127 and 7: the whole domain the kernels use it on.  A short chain of
// three dependent operations instead of the division's, whose latency sits
// on the critical path of every wave that meets a guarded element.
W4A8_HD float quant_div_corrected(float x, float s, float r)
{
    const float t = fmaf(x, r, -0.0f);
    const float e = fmaf(-t, s, x);
    return fmaf(e, r, t);
}

// The rule with that quotient (s != 0); equals quant_code_div on the domain above.
W4A8_HD int quant_code_corrected(float x, float s, float r, float qmax)
{
    float q = roundf(quant_div_corrected(x, s, r));   // halves go away from zero
    q = fminf(fmaxf(q, -qmax), qmax);
    return (int)q;
}

// Guard width: v within this distance of an integer goes to the slow path.
#define W4A8_QUANT_GUARD 0x1p-14f

// Fast path, in parts: the scaled value, its distance to the nearest
// integer, the code, and whether a distance needs the division rule.
W4A8_HD float quant_fast_t(float x, float r) { return fmaf(x, r, -0.0f); }   // == x * r
W4A8_HD float quant_fast_resid(float t) { return fabsf(t - rintf(t)); }      // exact
W4A8_HD int quant_fast_code(float t) { return (int)rintf(t); }
W4A8_HD bool quant_fast_slow(float resid) { return resid > 0.5f - W4A8_QUANT_GUARD; }

// One element: code and guard (|x| <= amax of the slice, see above).
W4A8_HD int quant_code_fast(float x, float r, float qmax, bool &slow)
{
    (void)qmax;
    const float t = quant_fast_t(x, r);
    slow |= quant_fast_slow(quant_fast_resid(t));
    return quant_fast_code(t);
}

}  // namespace w4a8
