// Host build of the library's quantization rule (w4a8_int8_gemm_amd/csrc/quant_rule.h),
// so the CPU test suite can check the GPU kernels' fast path against the oracle
// on every fp16 input.  Test code only.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../w4a8_int8_gemm_amd/csrc/quant_rule.h"

extern "C" {

// Codes of x[0..n) with the kernels' scheme: fast path, division rule for guarded elements.
// Returns how many elements took the division rule.
int shim_quantize(const float *x, int n, float amax, float qmax, int8_t *q, float *scale_out)
{
    const float s = w4a8::quant_scale(amax, qmax);
    *scale_out = s;
    int slow_count = 0;
    if (s == 0.0f) {
        for (int i = 0; i < n; ++i)
            q[i] = 0;
        return 0;
    }
    const float r = 1.0f / s;
    for (int i = 0; i < n; ++i) {
        bool slow = false;
        int c = w4a8::quant_code_fast(x[i], r, qmax, slow);
        if (slow) {
            c = w4a8::quant_code_div(x[i], s, qmax);
            ++slow_count;
        }
        q[i] = (int8_t)c;
    }
    return slow_count;
}

// fp16 bits to float (exact), for the exhaustive checks.
static float h2f_bits(uint16_t h)
{
    const int e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else
        v = ldexpf((float)(m | 0x400), e - 25);
    return (h & 0x8000) ? -v : v;
}

// Every fp16 amax with bits in [lo, hi) (finite, positive) and every fp16 x
// with |x| <= amax, both signs: the corrected quotient against x / s (equal
// values) and the code it gives against the division rule.  Returns the number
// of mismatches; the first one's amax and x bits go to *bad_amax, *bad_x.
long shim_check_corrected(int lo, int hi, float qmax, int *bad_amax, int *bad_x)
{
    long bad = 0;
    for (int ab = lo; ab < hi; ++ab) {
        const float amax = h2f_bits((uint16_t)ab);
        const float s = w4a8::quant_scale(amax, qmax);
        const float r = 1.0f / s;
        for (int xb = 0; xb <= ab; ++xb) {
            for (int sign = 0; sign < 2; ++sign) {
                const float x = h2f_bits((uint16_t)(xb | (sign << 15)));
                const float want = x / s;
                const float got = w4a8::quant_div_corrected(x, s, r);
                // equal as values (a zero quotient may differ in sign only)
                const bool same = want == got &&
                                  w4a8::quant_code_corrected(x, s, r, qmax) ==
                                      w4a8::quant_code_div(x, s, qmax);
                if (!same) {
                    if (bad == 0) {
                        *bad_amax = ab;
                        *bad_x = xb | (sign << 15);
                    }
                    ++bad;
                }
            }
        }
    }
    return bad;
}

// The same domain with the uncorrected product t = fl32(x r) in place of the
// corrected quotient: how many quotients differ from x / s (the correction
// step is needed).
long shim_count_uncorrected(int lo, int hi, float qmax)
{
    long bad = 0;
    for (int ab = lo; ab < hi; ++ab) {
        const float amax = h2f_bits((uint16_t)ab);
        const float s = w4a8::quant_scale(amax, qmax);
        const float r = 1.0f / s;
        for (int xb = 0; xb <= ab; ++xb) {
            const float x = h2f_bits((uint16_t)xb);
            bad += (x / s) != fmaf(x, r, -0.0f);
        }
    }
    return bad;
}

// quant_scale against the plain division for every non-negative fp16 amax
// (zero, subnormals, normals, infinity): the number of bit-pattern mismatches.
long shim_check_scale(float qmax)
{
    long bad = 0;
    for (int ab = 0; ab <= 0x7C00; ++ab) {
        const float amax = h2f_bits((uint16_t)ab);
        const float want = amax / qmax;
        const float got = w4a8::quant_scale(amax, qmax);
        bad += memcmp(&want, &got, sizeof(float)) != 0;
    }
    return bad;
}

// The fast path alone, without the guard's fallback.
void shim_fast_only(const float *x, int n, float amax, float qmax, int8_t *q)
{
    const float s = w4a8::quant_scale(amax, qmax);
    const float r = 1.0f / s;
    for (int i = 0; i < n; ++i) {
        bool slow = false;
        q[i] = (int8_t)w4a8::quant_code_fast(x[i], r, qmax, slow);
    }
}
}
