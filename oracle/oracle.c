/*
 * CPU oracle for the W8A8 / W4A8 int8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition the GPU library is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never calls it and shares no code with it.
 *
 * Sources (web pages; sections named as printed on them):
 *  [P1] "Apple Silicon의 AI 한계치는 당신의 생각보다 높습니다" (molayo1419.me),
 *       section "INT8 TensorOps 커널 설계" (kernel design): the four-step
 *       pipeline -- a min/max reduction gives the scale factors, activations
 *       are mapped to INT8 with them, the INT8 GEMM accumulates in INT32, and
 *       the INT32 result is rescaled by the product of the activation and
 *       weight scales to an FP16 output.  Section "입도: Per-Tensor vs.
 *       Per-Channel vs. Per-Group" (granularity): per-group scales need
 *       grouped dequantization during accumulation.
 *  [P2] "cider: Apple Silicon M5 INT8 TensorOps ... W8A8 SDK"
 *       (discuss.pytorch.kr), section "cider의 양자화 모드와 적용 가능한 영역"
 *       (quantization modes): W8A8 = symmetric INT8 weights x per-token INT8
 *       activations; W4A8 = INT4 weights packed in uint8, unpacked before the
 *       INT8 matmul; per-channel / per-group gs=128 / gs=64 variants.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - symmetric scales, s = fl32(amax / qmax) with qmax = 127 (int8) or 7 (int4);
 *  - codes are round-half-away-from-zero of fl32(x / s) (true IEEE division),
 *    clamped to [-qmax, qmax]; an all-zero slice gets s = 0 and zero codes;
 *  - int4 codes are two's-complement nibbles, low nibble = even k, packed
 *    along K into uint8 [N, K/2];
 *  - groups are contiguous slices of gs elements along K starting at k = 0;
 *  - the fp16 output is the IEEE round-to-nearest-even of the fp64 value.
 *
 * Floating point: the quantizer runs in fp32 because the scale rule fixes
 * that precision (the code is an integer decided by an fp32 division, and the
 * GPU takes the same decision in the same precision).  The rescale epilogue
 * runs in fp64 and is rounded once to fp16.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -fno-fast-math
 *        -ffp-contract=off oracle.c -lm   (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* -------------------------------------------------------------------------
 * IEEE binary16 <-> binary64.  Written from the format definition: 1 sign
 * bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 holds
 * subnormals (value = fraction * 2^-24).
 * ---------------------------------------------------------------------- */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* Round a binary64 value to the nearest binary16, ties to even, in one step
 * (no intermediate binary32, so there is no double rounding).  The scalings
 * by powers of two are exact; rint() rounds to nearest even in the default
 * rounding mode. */
uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: count units of 2^-24; 1024 units is the smallest
         * normal, whose bit pattern is also 1024 (0x0400). */
        double units = rint(ldexp(a, 24));
        return sign | (uint16_t)units;
    }
    int E;
    frexp(a, &E);               /* a in [2^(E-1), 2^E) */
    int e = E - 1;
    double mant = rint(ldexp(a, 10 - e));   /* in [1024, 2048] */
    if (mant == 2048.0) {
        mant = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7c00;   /* overflow rounds to infinity */
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(mant - 1024.0);
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set that number (timing runs measure the oracle on one thread and on all). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* -------------------------------------------------------------------------
 * Symmetric quantization of fp16 rows ([P1] kernel design, steps 1-2;
 * [P2] modes table).  For each row r and each slice g of `glen` contiguous
 * elements (glen = K when gs == 0, i.e. one scale per row):
 *     amax = max |x|                       (exact in fp32)
 *     s    = fl32(amax / qmax)
 *     q    = clamp(round_half_away(fl32(x / s)), -qmax, qmax)
 * Used for per-token activations (qmax 127), per-output-channel and
 * per-group int8 weights (qmax 127) and per-group int4 weights (qmax 7).
 * Scales are written row-major [rows, K/glen].  Returns 0, or -1 on a
 * non-finite input or a K that gs does not divide.
 * ---------------------------------------------------------------------- */
int oracle_quantize_sym(const uint16_t *x, int64_t rows, int64_t K, int64_t gs,
                        int32_t qmax, int8_t *q, float *s)
{
    int64_t glen = gs > 0 ? gs : K;
    if (glen <= 0 || K % glen != 0)
        return -1;
    int64_t G = K / glen;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *xs = x + r * K + g * glen;
            int8_t *qs = q + r * K + g * glen;
            float amax = 0.0f;
            for (int64_t k = 0; k < glen; ++k) {
                float v = (float)oracle_f16_to_f64(xs[k]);
                if (!isfinite(v))
                    bad = 1;
                float a = fabsf(v);
                if (a > amax)
                    amax = a;
            }
            float scale = amax / (float)qmax;
            s[r * G + g] = scale;
            for (int64_t k = 0; k < glen; ++k) {
                int8_t code = 0;
                if (scale != 0.0f) {
                    float t = (float)oracle_f16_to_f64(xs[k]) / scale;
                    float rt = roundf(t);   /* C roundf: halves go away from zero */
                    if (rt > (float)qmax)
                        rt = (float)qmax;
                    if (rt < (float)-qmax)
                        rt = (float)-qmax;
                    code = (int8_t)rt;
                }
                qs[k] = code;
            }
        }
    }
    return bad ? -1 : 0;
}

/* Pack int4 codes [N, K] (values in [-8, 7]) two per byte along K:
 * byte[n, j] = (code[n, 2j] & 0xF) | ((code[n, 2j+1] & 0xF) << 4). */
int oracle_pack_int4(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    if (K % 2 != 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t lo = (uint8_t)codes[n * K + 2 * j] & 0xF;
            uint8_t hi = (uint8_t)codes[n * K + 2 * j + 1] & 0xF;
            packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
    return 0;
}

/* Inverse of oracle_pack_int4: a nibble v >= 8 stands for v - 16. */
int oracle_unpack_int4(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    if (K % 2 != 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = packed[n * (K / 2) + j];
            int lo = b & 0xF, hi = b >> 4;
            codes[n * K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            codes[n * K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
    return 0;
}

/* -------------------------------------------------------------------------
 * int8 x int8 products with integer accumulation ([P1] kernel design,
 * step 3).  A is [M, K], B is [N, K] (both K-contiguous); the result is
 * C[m, n] = sum_k A[m, k] * B[n, k].  Sums are formed in int64 and stored as
 * int32; returns -1 if any sum falls outside the int32 range.
 * ---------------------------------------------------------------------- */
int oracle_gemm_i32(const int8_t *A, const int8_t *B, int64_t M, int64_t N, int64_t K,
                    int32_t *C)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
            if (acc > INT32_MAX || acc < INT32_MIN)
                bad = 1;
            C[m * N + n] = (int32_t)acc;
        }
    return bad ? -1 : 0;
}

/* Per-group partial sums ([P1] granularity section: grouped dequantization
 * during accumulation): P[g, m, n] = sum over k in group g of A[m,k]*B[n,k],
 * groups being contiguous slices of gs along K.  P is [G, M, N]. */
int oracle_gemm_partials(const int8_t *A, const int8_t *B, int64_t M, int64_t N, int64_t K,
                         int64_t gs, int32_t *P)
{
    if (gs <= 0 || K % gs != 0)
        return -1;
    int64_t G = K / gs;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < G; ++g) {
                int64_t acc = 0;
                for (int64_t k = g * gs; k < (g + 1) * gs; ++k)
                    acc += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
                P[(g * M + m) * N + n] = (int32_t)acc;   /* |acc| <= gs*127^2, far inside int32 */
            }
    return 0;
}

/* -------------------------------------------------------------------------
 * Rescale epilogues ([P1] kernel design, step 4).  fp64 arithmetic, one
 * final rounding to fp16 (round to nearest even).
 * ---------------------------------------------------------------------- */

/* Per-channel: Y[m, n] = fp16( C[m,n] * sa[m] * sw[n] ).  While |C| < 2^29
 * (any K up to 33 000) the product C*sa has at most 29 + 24 significant bits
 * and is exact in fp64, so the value before the fp16 rounding carries a
 * single fp64 rounding. */
void oracle_epilogue_pc(const int32_t *C, const float *sa, const float *sw, int64_t M,
                        int64_t N, uint16_t *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)C[m * N + n] * (double)sa[m] * (double)sw[n];
            Y[m * N + n] = oracle_f64_to_f16(v);
        }
}

/* Per-group: Y[m, n] = fp16( sum_g P[g,m,n] * sa[m,g] * sw[n,g] ), with
 * sa [M, G] and sw [N, G].  T[m, n] = sum_g |P * sa * sw| is the magnitude
 * sum that bounds any summation-order difference. */
void oracle_epilogue_pg(const int32_t *P, const float *sa, const float *sw, int64_t M,
                        int64_t N, int64_t G, uint16_t *Y, double *T)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double term = (double)P[(g * M + m) * N + n] * (double)sa[m * G + g] *
                              (double)sw[n * G + g];
                acc += term;
                mag += fabs(term);
            }
            Y[m * N + n] = oracle_f64_to_f16(acc);
            if (T)
                T[m * N + n] = mag;
        }
}

/* W4A8: per-token activation scale sa [M], per-group int4 weight scales
 * sw [N, G]:  Y[m, n] = fp16( sa[m] * sum_g P[g,m,n] * sw[n,g] ). */
void oracle_epilogue_w4a8(const int32_t *P, const float *sa, const float *sw, int64_t M,
                          int64_t N, int64_t G, uint16_t *Y, double *T)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double term = (double)P[(g * M + m) * N + n] * (double)sw[n * G + g];
                acc += term;
                mag += fabs(term);
            }
            Y[m * N + n] = oracle_f64_to_f16((double)sa[m] * acc);
            if (T)
                T[m * N + n] = fabs((double)sa[m]) * mag;
        }
}

/* -------------------------------------------------------------------------
 * Weight-only int8 product, the comparison baseline of the cider post's
 * latency table (section on its performance results): activations stay
 * fp16, weights are the int8 codes with per-channel scales:
 *     Y[m, n] = fp16( sw[n] * sum_k x[m,k] * wq[n,k] ),
 * the sum in binary64 (each product is exact: 11 x 8 significant bits), the
 * scale applied once in binary64, one rounding to fp16.  T[m, n] = sw[n] *
 * sum_k |x[m,k] * wq[n,k]| bounds the accumulation error of any fp32 order.
 * ---------------------------------------------------------------------- */
void oracle_w8a16(const uint16_t *X, const int8_t *W, const float *sw, int64_t M, int64_t N,
                  int64_t K, uint16_t *Y, double *T)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = oracle_f16_to_f64(X[m * K + k]) * (double)W[n * K + k];
                s += p;
                a += fabs(p);
            }
            Y[m * N + n] = oracle_f64_to_f16(s * (double)sw[n]);
            T[m * N + n] = a * (double)sw[n];
        }
    }
}

/* Weight-only int4 product, the latency table's other baseline: each int4
 * code (unpacked, [N, K]) is dequantized with its group's scale to fp16 as
 * fp16(fl32(code * sw[n, k / gs])) -- an fp32 multiply, then one rounding to
 * fp16 -- and Y[m, n] = fp16( sum_k x[m,k] * w[n,k] ), the sum in binary64
 * (each product of two fp16 values is exact), rounded once.  T[m, n] =
 * sum_k |x[m,k] * w[n,k]|. */
void oracle_w4a16(const uint16_t *X, const int8_t *codes, const float *sw, int64_t M, int64_t N,
                  int64_t K, int64_t gs, uint16_t *Y, double *T)
{
    const int64_t G = K / gs;
    double *Wd = (double *)malloc((size_t)(N * K) * sizeof(double));
    if (!Wd)
        return;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const float p = (float)codes[n * K + k] * sw[n * G + k / gs];
            Wd[n * K + k] = oracle_f16_to_f64(oracle_f64_to_f16((double)p));
        }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = oracle_f16_to_f64(X[m * K + k]) * Wd[n * K + k];
                s += p;
                a += fabs(p);
            }
            Y[m * N + n] = oracle_f64_to_f16(s);
            T[m * N + n] = a;
        }
    }
    free(Wd);
}
