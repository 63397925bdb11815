// Decode (M = 1) int8 matrix-vector product with the activation quantization
// fused in.  The "cider" post's path-selection section sends a single token to
// an INT8 matrix-vector kernel; its file list names a per-channel W8A8 MV.
// Decode reads every weight once, so the kernel is bound by HBM bandwidth
// (Apple-silicon essay, section on MLX and the prefill bottleneck: decode is
// memory-bandwidth bound).
//
// Each workgroup loads its share of the token (16-byte loads held in
// registers), then issues its weight-row loads (LPR lanes per row, up to CPL
// chunks per lane in flight), then derives the token's scale and codes from
// the registers while the weights stream in -- loads complete in issue order,
// so the token's data is waited for without waiting for the weights; every
// workgroup reaches the same codes because the rule is deterministic --
// stages the codes in LDS, and finishes with int8 dot products
// (v_dot4_i32_i8) and a lane reduction.  The rescale uses
// the GEMM epilogue's operation order, so results equal the GEMM path at M=1.
#include "kernels.hpp"

namespace w4a8 {

namespace {

template <int LPR, int CPL, int XCH>
__global__ __launch_bounds__(256) void int8_mv_kernel(const uint16_t *__restrict__ x,
                                                      const int8_t *__restrict__ w,
                                                      const float *__restrict__ sw,
                                                      uint16_t *__restrict__ y, int N, int K,
                                                      int8_t *__restrict__ xq_out,
                                                      float *__restrict__ xs_out)
{
    extern __shared__ __attribute__((aligned(16))) int8_t xq_s[];   // K bytes
    __shared__ uint32_t red[4];
    constexpr int RPB = 256 / LPR;                  // rows per workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x * RPB + tid / LPR;
    const int lr = tid % LPR;
    const int nch = K >> 4;                         // 16-byte chunks per weight row
    const bool row_ok = n < N;
    const uint4 *wr = reinterpret_cast<const uint4 *>(w + (int64_t)min(n, N - 1) * K);

    // 1. this thread's chunks of the token (8 fp16 each): c = tid + 256 j
    const uint4 *xr = reinterpret_cast<const uint4 *>(x);
    const int nx = K >> 3;
    uint4 xv[XCH];
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = tid + 256 * j;
        xv[j] = c < nx ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
    }

    // 2. first batch of weight loads in flight
    uint4 wv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        wv[j] = (c < nch) ? load_nt(wr + c) : make_uint4(0u, 0u, 0u, 0u);
    }

    // 3. the token's amax (reduction over the workgroup)
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < XCH; ++j)
        m = max(m, absmax_bits8(xv[j]));
    m = group_max_u32<64>(m);
    if (lane == 0)
        red[wave] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float s = quant_scale(h2f((uint16_t)m), 127.0f);
    const float r = 1.0f / s;

    // 4. codes into LDS (workgroup 0 also exports them when asked)
    const bool exporter = (blockIdx.x == 0);
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = tid + 256 * j;
        if (c < nx) {
            const uint2 q = quant_chunk8(xv[j], s, r, 127.0f);
            *reinterpret_cast<uint2 *>(xq_s + c * 8) = q;
            if (exporter && xq_out)
                *reinterpret_cast<uint2 *>(xq_out + c * 8) = q;
        }
    }
    if (exporter && tid == 0 && xs_out)
        xs_out[0] = s;
    __syncthreads();

    // 5. int8 dot products, then a reduction over the row's lanes
    int acc = 0;
    for (int base = 0;; base += LPR * CPL) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = base + lr + LPR * j;
            if (c < nch) {
                const uint4 q = *reinterpret_cast<const uint4 *>(xq_s + c * 16);
                acc = __builtin_amdgcn_sdot4((int)wv[j].x, (int)q.x, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wv[j].y, (int)q.y, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wv[j].z, (int)q.z, acc, false);
                acc = __builtin_amdgcn_sdot4((int)wv[j].w, (int)q.w, acc, false);
            }
        }
        const int next = base + LPR * CPL;
        if (next >= nch)
            break;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = next + lr + LPR * j;
            wv[j] = (c < nch) ? load_nt(wr + c) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    acc = group_sum_i32<LPR>(acc);
    if (lr == 0 && row_ok)
        y[n] = f2h(rescale_pc(acc, s, sw[n]));
}

template <int LPR, int CPL, int XCH>
void launch(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int N, int K,
            int8_t *xq_out, float *xs_out, hipStream_t st)
{
    constexpr int RPB = 256 / LPR;
    const unsigned blocks = (unsigned)((N + RPB - 1) / RPB);
    hipLaunchKernelGGL((int8_mv_kernel<LPR, CPL, XCH>), dim3(blocks), dim3(256), (size_t)K, st, x,
                       w, sw, y, N, K, xq_out, xs_out);
}

// Token chunks per thread: K / 8 chunks over 256 threads.
template <int LPR, int CPL>
void launch_x(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int N, int K,
              int8_t *xq_out, float *xs_out, hipStream_t st)
{
    const int xch = (K / 8 + 255) / 256;
    if constexpr (LPR == 16) {          // K <= 4096: at most two chunks
        if (xch <= 1)
            launch<LPR, CPL, 1>(x, w, sw, y, N, K, xq_out, xs_out, st);
        else
            launch<LPR, CPL, 2>(x, w, sw, y, N, K, xq_out, xs_out, st);
    } else {                            // 4096 < K <= 32768: 3 to 16 chunks
        if (xch <= 4)
            launch<LPR, CPL, 4>(x, w, sw, y, N, K, xq_out, xs_out, st);
        else if (xch <= 8)
            launch<LPR, CPL, 8>(x, w, sw, y, N, K, xq_out, xs_out, st);
        else
            launch<LPR, CPL, 16>(x, w, sw, y, N, K, xq_out, xs_out, st);
    }
}

}  // namespace

void launch_int8_mv(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int N,
                    int K, int8_t *xq_out, float *xs_out, hipStream_t st)
{
    const int nch = K / 16;
    if (nch <= 16 * 4)
        launch_x<16, 4>(x, w, sw, y, N, K, xq_out, xs_out, st);
    else if (nch <= 16 * 8)
        launch_x<16, 8>(x, w, sw, y, N, K, xq_out, xs_out, st);
    else if (nch <= 16 * 10)
        launch_x<16, 10>(x, w, sw, y, N, K, xq_out, xs_out, st);
    else if (nch <= 16 * 16)
        launch_x<16, 16>(x, w, sw, y, N, K, xq_out, xs_out, st);
    else
        launch_x<64, 16>(x, w, sw, y, N, K, xq_out, xs_out, st);
}

}  // namespace w4a8
