// Host build of the library's quantization rule (w4a8_int8_gemm_amd/csrc/quant_rule.h),
// so the CPU test suite can check the GPU kernels' fast path against the oracle
// on every fp16 input.  Test code only.
#include <stdint.h>

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
