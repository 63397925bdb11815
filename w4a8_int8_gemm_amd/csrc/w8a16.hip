// Weight-only GEMMs (W8A16, W4A16), the comparison paths of the "cider"
// post's latency table (section on its performance results: per-channel
// W8A8 against MLX's weight-only int8 and int4 products at N=10240,
// K=2560).  Activations stay fp16 and are multiplied on the fp16 matrix
// cores with fp32 accumulation:
//     W8A16: y[m, n] = fp16( w_scale[n] * sum_k x[m,k] * wq[n,k] ),
//            the int8 codes turned into fp16 exactly (|code| <= 128);
//     W4A16: y[m, n] = fp16( sum_k x[m,k] * fp16(fl32(code[n,k] * w_scale[n,g])) ),
//            each int4 code dequantized with its group's scale to fp16
//            before the product (weights packed as for w4a8_gemm).
//
// Design (a plain comparison kernel, not tuned like the int8 paths):
//  * 128 x 128 output tiles, four waves of 64 x 64, v_mfma_f32_32x32x16_f16
//    with the weights as the first operand, so a lane holds one output row m
//    and runs of four consecutive columns n (8-byte fp16 stores).
//  * K advances 64 at a time through two LDS buffers; both operands sit in
//    LDS as fp16 rows of 128 bytes with the 16-byte chunks XOR-swizzled per
//    row (conflict-free 16-byte fragment reads).  The next stage's global
//    loads are in flight while the current stage is multiplied; the weights
//    are converted to fp16 when they are written to LDS.
#include "kernels.hpp"

namespace w4a8 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int TB = 128;          // tile rows (m) and columns (n)
constexpr int KS = 64;           // k per stage: 128 bytes of fp16 per row

// Physical 16-byte chunk of logical chunk c (0..7) in a 128-byte LDS row r:
// sixteen consecutive rows read at one logical chunk hit distinct banks.
__device__ __forceinline__ int swz16(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Four signed bytes to four fp16 values, exactly: byte b + 128 is placed
// under the exponent byte 0x64 (fp16 1024 + (b + 128)), then 1152 is
// subtracted in fp16 (exact, the result is the integer b).
__device__ __forceinline__ uint2 int8x4_to_half4(uint32_t v)
{
    const uint32_t u = v ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const h2 k = {(_Float16)1152.0f, (_Float16)1152.0f};
    const h2 a = __builtin_bit_cast(h2, lo) - k;
    const h2 b = __builtin_bit_cast(h2, hi) - k;
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Eight packed int4 codes (one dword, low nibble = even k, two's-complement
// nibbles) dequantized with scale s to fp16, in k order: a nibble XOR 8 is
// u = code + 8, and fma(u, s, -8 s) rounds the exact code * s once, i.e.
// gives fl32(code * s); then fp16.
__device__ __forceinline__ uint4 int4x8_dequant(uint32_t v, float s)
{
    const uint32_t lo = (v & 0x0f0f0f0fu) ^ 0x08080808u;          // k = 0, 2, 4, 6
    const uint32_t hi = ((v >> 4) & 0x0f0f0f0fu) ^ 0x08080808u;   // k = 1, 3, 5, 7
    const float b = -8.0f * s;                        // exact (power of two)
    float d[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[2 * i] = fmaf((float)((lo >> (8 * i)) & 0xffu), s, b);
        d[2 * i + 1] = fmaf((float)((hi >> (8 * i)) & 0xffu), s, b);
    }
    return make_uint4(pack_h2(d[0], d[1]), pack_h2(d[2], d[3]), pack_h2(d[4], d[5]),
                      pack_h2(d[6], d[7]));
}

template <bool INT4>
__global__ __launch_bounds__(256) void w8a16_kernel(const uint16_t *__restrict__ x,
                                                    const void *__restrict__ wv,
                                                    const float *__restrict__ sw,
                                                    uint16_t *__restrict__ y, int M, int N, int K,
                                                    int gs)
{
    const int8_t *__restrict__ w = static_cast<const int8_t *>(wv);
    const uint8_t *__restrict__ w4 = static_cast<const uint8_t *>(wv);
    const int G = INT4 ? K / gs : 1;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][TB * 128];
    __shared__ __attribute__((aligned(16))) uint8_t ws[2][TB * 128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;          // 64 x 64 wave tile (n, m)
    const int n0 = blockIdx.x * TB, m0 = blockIdx.y * TB;
    const int nst = K / KS;

    // global loads of one stage: X 1024 chunks of 16 bytes (4 per thread),
    // W 512 chunks of 16 int8 (2 per thread) or 256 chunks of 32 packed
    // int4 codes (one per thread, with its group's scale); rows past the
    // end read zeros
    uint4 xr[4], wr[2];
    float wsc = 0.0f;
    auto load = [&](int s) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)s * KS;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int c = tid + 256 * p, r = c >> 3, ch = c & 7;
            const int m = m0 + r;
            xr[p] = m < M ? *reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k0 + ch * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
        if constexpr (INT4) {
            const int r = tid >> 1, half = tid & 1;  // 32 codes: k0 + 32 half .. + 31
            const int n = n0 + r;
            const int64_t kc = k0 + 32 * half;
            wr[0] = n < N ? *reinterpret_cast<const uint4 *>(w4 + (int64_t)n * (K / 2) + kc / 2)
                          : make_uint4(0u, 0u, 0u, 0u);
            wsc = n < N ? sw[(int64_t)n * G + kc / gs] : 0.0f;
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int c = tid + 256 * p, r = c >> 2, ch = c & 3;
                const int n = n0 + r;
                wr[p] = n < N ? *reinterpret_cast<const uint4 *>(w + (int64_t)n * K + k0 + ch * 16)
                              : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int c = tid + 256 * p, r = c >> 3, ch = c & 7;
            *reinterpret_cast<uint4 *>(&xs[buf][r * 128 + swz16(r, ch) * 16]) = xr[p];
        }
        if constexpr (INT4) {
            const int r = tid >> 1, half = tid & 1;  // 32 codes -> fp16 chunks 4 half .. 4 half + 3
            const uint32_t q[4] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4 *>(&ws[buf][r * 128 + swz16(r, 4 * half + i) * 16]) =
                    int4x8_dequant(q[i], wsc);
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int c = tid + 256 * p, r = c >> 2, ch = c & 3;   // 16 codes -> fp16 chunks 2ch, 2ch+1
                const uint2 a = int8x4_to_half4(wr[p].x), b = int8x4_to_half4(wr[p].y);
                const uint2 d = int8x4_to_half4(wr[p].z), e = int8x4_to_half4(wr[p].w);
                *reinterpret_cast<uint4 *>(&ws[buf][r * 128 + swz16(r, 2 * ch) * 16]) =
                    make_uint4(a.x, a.y, b.x, b.y);
                *reinterpret_cast<uint4 *>(&ws[buf][r * 128 + swz16(r, 2 * ch + 1) * 16]) =
                    make_uint4(d.x, d.y, e.x, e.y);
            }
        }
    };

    f16x acc[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            acc[j][i] = f16x{};

    // fragment of k-step t (16 k): row base + lane % 32, logical chunk
    // 2t + lane / 32 (eight fp16 values)
    const int lr = lane & 31, lh = lane >> 5;
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        if (s + 1 < nst)
            load(s + 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            h8 a[2], b[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + lr;
                a[j] = *reinterpret_cast<const h8 *>(&ws[buf][r * 128 + swz16(r, 2 * t + lh) * 16]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + lr;
                b[i] = *reinterpret_cast<const h8 *>(&xs[buf][r * 128 + swz16(r, 2 * t + lh) * 16]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[i], acc[j][i], 0, 0, 0);
        }
        if (s + 1 < nst) {
            store(buf ^ 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds row m of block (j, i) and columns
    // nb + 8g + 4 lh + 0..3 in elements 4g..4g+3
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + i * 32 + lr;
        if (m >= M)
            continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nb = n0 + wn * 64 + j * 32;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nb + 8 * g + 4 * lh;
                if constexpr (INT4) {
                    if (vec && n + 3 < N) {
                        *reinterpret_cast<uint2 *>(y + (int64_t)m * N + n) =
                            make_uint2(pack_h2(acc[j][i][4 * g], acc[j][i][4 * g + 1]),
                                       pack_h2(acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                y[(int64_t)m * N + n + r] = f2h(acc[j][i][4 * g + r]);
                    }
                } else if (vec && n + 3 < N) {
                    const uint32_t p0 = pack_h2(acc[j][i][4 * g] * sw[n], acc[j][i][4 * g + 1] * sw[n + 1]);
                    const uint32_t p1 =
                        pack_h2(acc[j][i][4 * g + 2] * sw[n + 2], acc[j][i][4 * g + 3] * sw[n + 3]);
                    *reinterpret_cast<uint2 *>(y + (int64_t)m * N + n) = make_uint2(p0, p1);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            y[(int64_t)m * N + n + r] = f2h(acc[j][i][4 * g + r] * sw[n + r]);
                }
            }
        }
    }
}

// Decode (M = 1) form of the weight-only products: the token is staged in
// LDS as fp32, 16 lanes share a weight row (16-byte chunks, 16 int8 or 32
// int4 codes each, up to 8 chunks per lane in flight), products accumulate
// in fp32 and the row's lanes add their sums.  Weights are dequantized as in
// the GEMM (int8: exact, scale at the end; int4: fp16(fl32(code * s))).
template <bool INT4>
__global__ __launch_bounds__(256) void wo_mv_kernel(const uint16_t *__restrict__ x,
                                                    const void *__restrict__ wv,
                                                    const float *__restrict__ sw,
                                                    uint16_t *__restrict__ y, int N, int K, int gs)
{
    extern __shared__ __attribute__((aligned(16))) float xf[];   // K floats
    const int tid = threadIdx.x;
    for (int c = tid; c < K / 8; c += 256) {
        const uint4 v = *reinterpret_cast<const uint4 *>(x + c * 8);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xf[c * 8 + 2 * i] = h2f((uint16_t)(u[i] & 0xffffu));
            xf[c * 8 + 2 * i + 1] = h2f((uint16_t)(u[i] >> 16));
        }
    }
    __syncthreads();
    const int n = blockIdx.x * 16 + (tid >> 4), lr = tid & 15;
    const int nr = min(n, N - 1);
    constexpr int KPC = INT4 ? 32 : 16;               // codes per 16-byte chunk
    const int nch = K / KPC;
    const uint8_t *wr = static_cast<const uint8_t *>(wv) + (int64_t)nr * (K / (INT4 ? 2 : 1));
    const int G = INT4 ? K / gs : 1;
    float acc = 0.0f;
    for (int base = 0; base < nch; base += 16 * 8) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = base + lr + 16 * j;
            v[j] = c < nch ? *reinterpret_cast<const uint4 *>(wr + c * 16) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = base + lr + 16 * j;
            if (c >= nch)
                continue;
            const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            const float *xc = xf + c * KPC;
            if constexpr (INT4) {
                const float s = sw[(int64_t)nr * G + (c * KPC) / gs];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 h = int4x8_dequant(q[i], s);
                    const uint32_t hh[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(xc[8 * i + 2 * e], h2f((uint16_t)(hh[e] & 0xffffu)), acc);
                        acc = fmaf(xc[8 * i + 2 * e + 1], h2f((uint16_t)(hh[e] >> 16)), acc);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc = fmaf(xc[4 * i + e], (float)(int8_t)(q[i] >> (8 * e)), acc);
            }
        }
    }
    // sum over the row's 16 lanes
#pragma unroll
    for (int o = 8; o > 0; o >>= 1)
        acc += __shfl_xor(acc, o, 16);
    if (lr == 0 && n < N)
        y[n] = f2h(INT4 ? acc : acc * sw[n]);
}

}  // namespace

void launch_wo_mv(bool int4, const uint16_t *x, const void *w, const float *sw, int gs, uint16_t *y,
                  int N, int K, hipStream_t st)
{
    const unsigned blocks = (unsigned)((N + 15) / 16);
    const size_t lds = (size_t)K * sizeof(float);
    if (int4)
        hipLaunchKernelGGL(wo_mv_kernel<true>, dim3(blocks), dim3(256), lds, st, x, w, sw, y, N, K, gs);
    else
        hipLaunchKernelGGL(wo_mv_kernel<false>, dim3(blocks), dim3(256), lds, st, x, w, sw, y, N, K, 0);
}

void launch_w8a16(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int M, int N,
                  int K, hipStream_t st)
{
    const dim3 grid((unsigned)((N + TB - 1) / TB), (unsigned)((M + TB - 1) / TB));
    hipLaunchKernelGGL(w8a16_kernel<false>, grid, dim3(256), 0, st, x, (const void *)w, sw, y, M,
                       N, K, 0);
}

void launch_w4a16(const uint16_t *x, const uint8_t *w4, const float *sw, int gs, uint16_t *y, int M,
                  int N, int K, hipStream_t st)
{
    const dim3 grid((unsigned)((N + TB - 1) / TB), (unsigned)((M + TB - 1) / TB));
    hipLaunchKernelGGL(w8a16_kernel<true>, grid, dim3(256), 0, st, x, (const void *)w4, sw, y, M,
                       N, K, gs);
}

}  // namespace w4a8
