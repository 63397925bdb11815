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

    // 1. this thread's chunks of the token (8 fp16 each): c = tid + 256 j.
    // Indexes past the end are clamped to the last chunk, whose value then
    // goes unused (a repeated chunk leaves the amax as it is, and the codes
    // and dot products below skip it): no load sits under a branch, since a
    // branch around a load makes the compiler wait for every load in flight
    // where the paths join, and the token would then wait for the weights.
    const uint4 *xr = reinterpret_cast<const uint4 *>(x);
    const int nx = K >> 3;
    uint4 xv[XCH];
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = tid + 256 * j;
        xv[j] = xr[min(c, nx - 1)];
    }

    // 2. first batch of weight loads in flight
    uint4 wv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        wv[j] = load_nt(wr + min(c, nch - 1));
    }
    const float swn = sw[min(n, N - 1)];            // the row's scale, for the rescale

    // every load above is issued before any of the token's data is used
    __builtin_amdgcn_sched_barrier(0);

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
            wv[j] = load_nt(wr + min(c, nch - 1));
        }
    }
    acc = group_sum_i32<LPR>(acc);
    if (lr == 0 && row_ok)
        y[n] = f2h(rescale_pc(acc, s, swn));
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


// fp32 sum over groups of `width` consecutive lanes (16, 32 or 64), with
// the DPP moves of lane_reduce on the bit patterns (a lane a move does not
// reach takes +0).  The sum is in every lane of the group at widths 16 and
// 64, and in the group's upper 16 lanes at width 32 (so the group's last lane
// always holds it).
template <int width>
__device__ __forceinline__ float group_sum_f32(float v)
{
#define W4A8_DPPF(x, ctrl, rows) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctrl), (rows), 0xf, false))
    static_assert(width == 16 || width == 32 || width == 64, "reduction width");
    v += W4A8_DPPF(v, 0xb1, 0xf);
    v += W4A8_DPPF(v, 0x4e, 0xf);
    v += W4A8_DPPF(v, 0x141, 0xf);
    v += W4A8_DPPF(v, 0x140, 0xf);
    if constexpr (width == 32)
        v += W4A8_DPPF(v, 0x142, 0xa);             // row_bcast:15: rows 0, 2 into rows 1, 3
    if constexpr (width == 64) {
        v += W4A8_DPPF(v, 0x142, 0xa);
        v += W4A8_DPPF(v, 0x143, 0xc);
        v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    }
#undef W4A8_DPPF
    return v;
}

// Decode with per-group weight scales: the per-group W8A8 mode (the token is
// quantized per group of GS as well) and W4A8 (packed int4 weights, one
// scale for the token).  A 16-byte weight chunk (16 int8 or 32 int4 codes)
// lies inside one group; the CPG lanes holding the chunks of a group add
// their int32 dot products (exact), and the group's first lane folds the
// sum into its fp32 accumulator with the group's scales in the GEMM's
// operation order (fma of the sum with sa*sw, or with sw for int4); the
// row's lanes then add their accumulators.  int4 codes are used as
// 16 * code (the nibble moved into the high half of a byte), so the token's
// codes are staged split into even and odd k to meet the low and high
// nibbles of each weight byte; the factor 16 is undone at the end (exact).
template <bool INT4, int GS, int LPR, int CPL, int XCH, int NT>
__global__ __launch_bounds__(NT) void mv_group_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ w,
                                                       const float *__restrict__ sw,
                                                       uint16_t *__restrict__ y, int N, int K)
{
    // LDS: the token's codes (K bytes), then its per-group scales (per-group
    // mode, K/GS floats)
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    constexpr int NW = NT / 64;                     // waves per workgroup
    __shared__ uint32_t red[NW];
    constexpr int RPB = NT / LPR;                   // rows per workgroup
    constexpr int KPC = INT4 ? 32 : 16;             // k per 16-byte weight chunk
    constexpr int CPG = GS / KPC;                   // chunks per group
    static_assert(CPG == 2 || CPG == 4 || CPG == 8, "chunks per group");
    const int G = K / GS;
    int8_t *xq_s = smem;
    float *sa_s = reinterpret_cast<float *>(smem + K);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * RPB;
    const int rl = tid / LPR, lr = tid % LPR;
    const int n = n0 + rl;
    const int rowb = INT4 ? K / 2 : K;              // bytes per weight row
    const int nch = rowb >> 4;
    const uint4 *wr = reinterpret_cast<const uint4 *>(w + (int64_t)min(n, N - 1) * rowb);
    const float *swr = sw + (int64_t)min(n, N - 1) * G;    // the row's group scales
    const bool leader = lr % CPG == 0;              // first lane of its group's lanes

    // 1. this thread's chunks of the token (8 fp16 each): c = tid + 256 j,
    // loads clamped to the last chunk as in the per-channel kernel
    const uint4 *xr = reinterpret_cast<const uint4 *>(x);
    const int nx = K >> 3;
    uint4 xv[XCH];
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
        const int c = tid + NT * j;
        xv[j] = xr[min(c, nx - 1)];
    }

    // 2. first batch of weight loads in flight, with the group scales the
    // leading lanes fold them with
    uint4 wv[CPL];
    float swv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        wv[j] = load_nt(wr + min(c, nch - 1));
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        swv[j] = swr[min(c, nch - 1) / CPG];
    }

    __builtin_amdgcn_sched_barrier(0);

    // 3. the token's scale(s) and codes
    float s = 0.0f;                                 // the token's scale (int4)
    if constexpr (INT4) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < XCH; ++j)
            m = max(m, absmax_bits8(xv[j]));
        m = group_max_u32<64>(m);
        if (lane == 0)
            red[wave] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int i = 1; i < NW; ++i)
            m = max(m, red[i]);
        s = quant_scale(h2f((uint16_t)m), 127.0f);
        const float r = 1.0f / s;
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = tid + NT * j;
            if (c < nx) {
                // k 8c .. 8c+7 -> (even k, odd k): the order of the low and
                // high nibbles of the weight dword that covers them
                const uint2 q = quant_chunk8(xv[j], s, r, 127.0f);
                *reinterpret_cast<uint2 *>(xq_s + c * 8) =
                    make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x06040200u),
                               __builtin_amdgcn_perm(q.y, q.x, 0x07050301u));
            }
        }
    } else {
        // groups of GS / 8 consecutive threads share a group of the token
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = tid + NT * j;
            const uint32_t m = group_max_u32<GS / 8>(absmax_bits8(xv[j]));
            const float sg = quant_scale(h2f((uint16_t)m), 127.0f);
            const float r = 1.0f / sg;
            if (c < nx) {
                *reinterpret_cast<uint2 *>(xq_s + c * 8) = quant_chunk8(xv[j], sg, r, 127.0f);
                if (tid % (GS / 8) == 0)
                    sa_s[(c * 8) / GS] = sg;
            }
        }
    }
    __syncthreads();

    // 4. per chunk: int32 dot product, summed over the group's lanes, folded
    // by the group's first lane
    float acc = 0.0f;
    for (int base = 0;; base += LPR * CPL) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = base + lr + LPR * j;
            int p = 0;
            if (c < nch) {
                const uint4 v = wv[j];
                if constexpr (INT4) {
                    const uint4 q0 = *reinterpret_cast<const uint4 *>(xq_s + c * 32);
                    const uint4 q1 = *reinterpret_cast<const uint4 *>(xq_s + c * 32 + 16);
                    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
                    const uint32_t qe[4] = {q0.x, q0.z, q1.x, q1.z}, qo[4] = {q0.y, q0.w, q1.y, q1.w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        p = __builtin_amdgcn_sdot4((int)((wd[d] << 4) & 0xf0f0f0f0u), (int)qe[d], p, false);
                        p = __builtin_amdgcn_sdot4((int)(wd[d] & 0xf0f0f0f0u), (int)qo[d], p, false);
                    }
                } else {
                    const uint4 q = *reinterpret_cast<const uint4 *>(xq_s + c * 16);
                    p = __builtin_amdgcn_sdot4((int)v.x, (int)q.x, p, false);
                    p = __builtin_amdgcn_sdot4((int)v.y, (int)q.y, p, false);
                    p = __builtin_amdgcn_sdot4((int)v.z, (int)q.z, p, false);
                    p = __builtin_amdgcn_sdot4((int)v.w, (int)q.w, p, false);
                }
            }
            p = group_sum_i32<CPG>(p);              // every lane of the wave takes part
            if (leader && c < nch) {
                const float sc = INT4 ? swv[j] : sa_s[c / CPG] * swv[j];
                acc = fmaf((float)p, sc, acc);
            }
        }
        const int next = base + LPR * CPL;
        if (next >= nch)
            break;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = next + lr + LPR * j;
            wv[j] = load_nt(wr + min(c, nch - 1));
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = next + lr + LPR * j;
            swv[j] = swr[min(c, nch - 1) / CPG];
        }
    }
    acc = group_sum_f32<LPR>(acc);
    if (lr == LPR - 1 && n < N)
        y[n] = f2h(INT4 ? acc * (s * 0.0625f) : acc);
}

template <bool INT4, int GS, int LPR, int CPL, int XCH, int NT = 256>
void launch_group(const uint16_t *x, const uint8_t *w, const float *sw, uint16_t *y, int N,
                  int K, hipStream_t st)
{
    constexpr int RPB = NT / LPR;
    const unsigned blocks = (unsigned)((N + RPB - 1) / RPB);
    const size_t lds = (size_t)K + sizeof(float) * (INT4 ? 0 : K / GS);
    hipLaunchKernelGGL((mv_group_kernel<INT4, GS, LPR, CPL, XCH, NT>), dim3(blocks), dim3(NT), lds,
                       st, x, w, sw, y, N, K);
}

// Workgroups of NT = 512 or 768 threads (2-3x the rows of a 256-thread
// workgroup, so the token is quantized that much less often and each thread
// quantizes fewer of its chunks).  Taken for int4 where the workgroups then
// fit one round over the compute units, and for int8 rows up to K = 8192
// (measured, warm / cold us: int4 4096 x 12288 9.4 / 10.8 -> 8.4 / 9.1 at 512
// threads, int4 6144 x 4096 5.1 / 5.0 -> 4.5 / 4.9 at 768, int8 gs=128 4096 x
// 4096 5.0 / 4.5 -> 4.5 / 3.9 and 6144 x 4096 6.1 -> 5.4 warm at 512; int4 at
// 6144 rows with 512 threads, 1.5 workgroups per compute unit, ran 5-25 %
// slower, int8 at K = 14336 4 % slower).  Token chunks per thread by K.
template <bool INT4, int GS, int LPR, int NT>
void launch_group_nt(const uint16_t *x, const uint8_t *w, const float *sw, uint16_t *y, int N,
                     int K, hipStream_t st)
{
    const int nch = (INT4 ? K / 2 : K) / 16;
    const int xch = (K / 8 + NT - 1) / NT;
    if (nch <= LPR * 4 && xch <= 1)
        launch_group<INT4, GS, LPR, 4, 1, NT>(x, w, sw, y, N, K, st);
    else if (nch <= LPR * 8 && xch <= 1)
        launch_group<INT4, GS, LPR, 8, 1, NT>(x, w, sw, y, N, K, st);
    else if (xch <= 1)
        launch_group<INT4, GS, LPR, 16, 1, NT>(x, w, sw, y, N, K, st);
    else if (xch <= 2)
        launch_group<INT4, GS, LPR, 16, 2, NT>(x, w, sw, y, N, K, st);
    else if (xch <= 4)
        launch_group<INT4, GS, LPR, 16, 4, NT>(x, w, sw, y, N, K, st);
    else
        launch_group<INT4, GS, LPR, 16, 8, NT>(x, w, sw, y, N, K, st);
}

// 16 lanes per row (16 rows per workgroup, so the token's quantization is
// shared by 16 rows at any K) while that gives at least two workgroups per
// compute unit; fewer rows take 64 lanes per row (int8; 4 rows per
// workgroup) or 32 (int4, whose chunks carry twice the codes; 8 rows per
// workgroup), so that every compute unit still has several row streams in
// flight (measured: int8 4096 x 14336 16.7 us instead of 19.5; int4 rows
// lost 25-35 % at 64 lanes).  Chunks in flight per lane by the row's 16-byte chunks (rows longer
// than LPR * 16 chunks take several passes); token chunks per thread by K.
template <bool INT4, int GS, int LPR>
void launch_group_l(const uint16_t *x, const uint8_t *w, const float *sw, uint16_t *y, int N,
                    int K, hipStream_t st)
{
    const int nch = (INT4 ? K / 2 : K) / 16;
    if (K <= 4096) {
        if (nch <= LPR * 4)
            launch_group<INT4, GS, LPR, 4, 2>(x, w, sw, y, N, K, st);
        else if (nch <= LPR * 8)
            launch_group<INT4, GS, LPR, 8, 2>(x, w, sw, y, N, K, st);
        else
            launch_group<INT4, GS, LPR, 16, 2>(x, w, sw, y, N, K, st);
    } else if (K <= 8192) {
        launch_group<INT4, GS, LPR, 16, 4>(x, w, sw, y, N, K, st);
    } else if (K <= 16384) {
        launch_group<INT4, GS, LPR, 16, 8>(x, w, sw, y, N, K, st);
    } else {
        launch_group<INT4, GS, LPR, 16, 16>(x, w, sw, y, N, K, st);
    }
}

template <bool INT4, int GS>
void launch_group_k(const uint16_t *x, const uint8_t *w, const float *sw, uint16_t *y, int N,
                    int K, int cu, hipStream_t st)
{
    if (N >= 16 * 2 * cu)
        launch_group_l<INT4, GS, 16>(x, w, sw, y, N, K, st);
    else if (INT4 && (N + 15) / 16 <= cu)
        launch_group_nt<INT4, GS, 32, 512>(x, w, sw, y, N, K, st);
    else if (INT4 && (N + 23) / 24 <= cu)
        launch_group_nt<INT4, GS, 32, 768>(x, w, sw, y, N, K, st);
    else if (INT4)
        launch_group_l<INT4, GS, 32>(x, w, sw, y, N, K, st);
    else if (K <= 8192)
        launch_group_nt<INT4, GS, 64, 512>(x, w, sw, y, N, K, st);
    else
        launch_group_l<INT4, GS, 64>(x, w, sw, y, N, K, st);
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

namespace {

// Few tokens, per-channel scales: the GEMM's arithmetic in the decode
// kernel's shape.  The weight rows are streamed whole (LPR lanes per row, CPL
// 16-byte chunks per lane in flight, RPT rows per lane group) and each chunk
// is dotted with the codes of all M <= MT tokens, staged in LDS; per token one
// exact int32 sum per row, then the GEMM epilogue's rescale, so the result
// equals the GEMM's bit for bit.
template <int MT, int LPR, int CPL, int RPT>
__global__ __launch_bounds__(256) void few_pc_kernel(const int8_t *__restrict__ xq,
                                                     const float *__restrict__ xs,
                                                     const int8_t *__restrict__ w,
                                                     const float *__restrict__ sw,
                                                     uint16_t *__restrict__ y, int M, int N, int K)
{
    extern __shared__ __attribute__((aligned(16))) int8_t xq_s[];   // M * K bytes
    constexpr int RPB = 256 / LPR;                  // rows per pass of the workgroup
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int nch = K >> 4;
    int n[RPT];
    const uint4 *wr[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        n[r] = blockIdx.x * (RPB * RPT) + r * RPB + tid / LPR;
        wr[r] = reinterpret_cast<const uint4 *>(w + (int64_t)min(n[r], N - 1) * K);
    }
    // Loads in the order their data is needed (they complete in issue order):
    // the tokens' codes (held in registers while K <= 4096, i.e. at most MT
    // chunks per thread), then the weight rows, then the scales for the
    // rescale.  Indexes past the end are clamped and their values unused, so
    // that no load sits under a branch (the compiler would wait for every
    // load in flight where the paths join).
    const int xch = (M * K) >> 4;
    // (native vector type: a struct copy would be folded into a memcpy at
    // the LDS store, after the weight loads)
    const v4u *xq4 = reinterpret_cast<const v4u *>(xq);
    constexpr int XQ = LPR == 16 ? MT : 1;
    v4u xqv[XQ];
    if constexpr (LPR == 16) {
#pragma unroll
        for (int j = 0; j < XQ; ++j)
            xqv[j] = xq4[min(tid + 256 * j, xch - 1)];
    }
    uint4 wv[RPT][CPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lr + LPR * j;
            wv[r][j] = load_nt(wr[r] + min(c, nch - 1));
        }
    float swn[RPT], xsv[MT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        swn[r] = sw[min(n[r], N - 1)];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        xsv[t] = xs[min(t, M - 1)];
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LPR == 16) {
        // a clamped index stores the last chunk's own value again
#pragma unroll
        for (int j = 0; j < XQ; ++j)
            reinterpret_cast<v4u *>(xq_s)[min(tid + 256 * j, xch - 1)] = xqv[j];
    } else {
        for (int c = tid; c < xch; c += 256)
            reinterpret_cast<v4u *>(xq_s)[c] = xq4[c];
    }
    __syncthreads();

    int acc[RPT][MT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
            acc[r][t] = 0;
    for (int base = 0;; base += LPR * CPL) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = base + lr + LPR * j;
            if (c < nch) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t < M) {
                        const uint4 q = *reinterpret_cast<const uint4 *>(xq_s + t * K + c * 16);
#pragma unroll
                        for (int r = 0; r < RPT; ++r) {
                            int a = acc[r][t];
                            a = __builtin_amdgcn_sdot4((int)wv[r][j].x, (int)q.x, a, false);
                            a = __builtin_amdgcn_sdot4((int)wv[r][j].y, (int)q.y, a, false);
                            a = __builtin_amdgcn_sdot4((int)wv[r][j].z, (int)q.z, a, false);
                            acc[r][t] = __builtin_amdgcn_sdot4((int)wv[r][j].w, (int)q.w, a, false);
                        }
                    }
                }
            }
        }
        const int next = base + LPR * CPL;
        if (next >= nch)
            break;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = next + lr + LPR * j;
                wv[r][j] = load_nt(wr[r] + min(c, nch - 1));
            }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                const int a = group_sum_i32<LPR>(acc[r][t]);
                if (lr == 0 && n[r] < N)
                    y[(int64_t)t * N + n[r]] = f2h(rescale_pc(a, xsv[t], swn[r]));
            }
        }
    }
}

template <int MT, int LPR, int CPL>
void launch_few(const int8_t *xq, const float *xs, const int8_t *w, const float *sw, uint16_t *y,
                int M, int N, int K, hipStream_t st)
{
    // two rows per lane group (each token chunk read from LDS serves both)
    // where it measured faster: four tokens at 64 lanes per row (K > 4096)
    constexpr int RPT = (MT == 4 && LPR == 64) ? 2 : 1;
    constexpr int RPB = 256 / LPR * RPT;
    const unsigned blocks = (unsigned)((N + RPB - 1) / RPB);
    hipLaunchKernelGGL((few_pc_kernel<MT, LPR, CPL, RPT>), dim3(blocks), dim3(256), (size_t)M * K, st,
                       xq, xs, w, sw, y, M, N, K);
}

// Few tokens, W4A8: the decode kernel's int4 row streaming (16 lanes per row;
// a 16-byte chunk holds 32 codes of one group) for M <= MT tokens quantized
// per token.  The tokens' codes are staged in LDS split into even and odd k,
// the order of the low and high nibbles of each weight byte; a nibble moved
// into the high half of its byte reads as 16 * code, so each group's int32
// dot product is 16 P_g, summed over the group's lanes and folded in fp32 by
// its first lane with the group's weight scale; the row's lanes then add
// their accumulators, and the 16 is undone with the token's scale (exact).
template <int MT, int GS, int CPL>
__global__ __launch_bounds__(256) void few_w4_kernel(const int8_t *__restrict__ xq,
                                                     const float *__restrict__ xs,
                                                     const uint8_t *__restrict__ w,
                                                     const float *__restrict__ sw,
                                                     uint16_t *__restrict__ y, int M, int N, int K)
{
    extern __shared__ __attribute__((aligned(16))) int8_t xq_s[];   // M * K bytes
    constexpr int LPR = 16, RPB = 256 / LPR;
    constexpr int CPG = GS / 32;                    // chunks per group
    static_assert(CPG == 2 || CPG == 4, "chunks per group");
    const int G = K / GS;
    const int tid = threadIdx.x;
    const int n = blockIdx.x * RPB + tid / LPR;
    const int lr = tid % LPR;
    const int nch = K >> 5;                         // 16-byte chunks per packed row
    const uint4 *wr = reinterpret_cast<const uint4 *>(w + (int64_t)min(n, N - 1) * (K / 2));
    const float *swr = sw + (int64_t)min(n, N - 1) * G;
    const bool leader = lr % CPG == 0;

    // Loads in the order their data is needed, none under a branch (as in
    // the per-channel few-token kernel): the tokens' codes, 8 k at a time
    // (in registers while K <= 4096: at most 2 MT pieces per thread), the
    // weight rows, their group scales and the tokens' scales.
    const int x8 = (M * K) >> 3;
    const uint2 *xq2 = reinterpret_cast<const uint2 *>(xq);
    constexpr bool XREG = CPL <= 8;                 // K <= 4096
    constexpr int XQ = XREG ? 2 * MT : 1;
    uint2 xqv[XQ];
    if constexpr (XREG) {
#pragma unroll
        for (int j = 0; j < XQ; ++j)
            xqv[j] = xq2[min(tid + 256 * j, x8 - 1)];
    }
    uint4 wv[CPL];
    float swv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        wv[j] = load_nt(wr + min(c, nch - 1));
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        swv[j] = swr[min(c, nch - 1) / CPG];
    }
    float xsv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        xsv[t] = xs[min(t, M - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // the codes into LDS as (even k, odd k)
    if constexpr (XREG) {
        // a clamped index stores the last piece's own value again
#pragma unroll
        for (int j = 0; j < XQ; ++j) {
            const uint2 q = xqv[j];
            reinterpret_cast<uint2 *>(xq_s)[min(tid + 256 * j, x8 - 1)] =
                make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x06040200u),
                           __builtin_amdgcn_perm(q.y, q.x, 0x07050301u));
        }
    } else {
        for (int c = tid; c < x8; c += 256) {
            const uint2 q = xq2[c];
            reinterpret_cast<uint2 *>(xq_s)[c] =
                make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x06040200u),
                           __builtin_amdgcn_perm(q.y, q.x, 0x07050301u));
        }
    }
    __syncthreads();

    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = 0.0f;
    for (int base = 0;; base += LPR * CPL) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = base + lr + LPR * j;
            const uint32_t wd[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < M) {
                    int p = 0;
                    if (c < nch) {
                        const int8_t *xt = xq_s + t * K + c * 32;
                        const uint4 q0 = *reinterpret_cast<const uint4 *>(xt);
                        const uint4 q1 = *reinterpret_cast<const uint4 *>(xt + 16);
                        const uint32_t qe[4] = {q0.x, q0.z, q1.x, q1.z};
                        const uint32_t qo[4] = {q0.y, q0.w, q1.y, q1.w};
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            p = __builtin_amdgcn_sdot4((int)((wd[d] << 4) & 0xf0f0f0f0u), (int)qe[d], p, false);
                            p = __builtin_amdgcn_sdot4((int)(wd[d] & 0xf0f0f0f0u), (int)qo[d], p, false);
                        }
                    }
                    p = group_sum_i32<CPG>(p);      // every lane of the wave takes part
                    if (leader && c < nch)
                        acc[t] = fmaf((float)p, swv[j], acc[t]);
                }
            }
        }
        const int next = base + LPR * CPL;
        if (next >= nch)
            break;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = next + lr + LPR * j;
            wv[j] = load_nt(wr + min(c, nch - 1));
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = next + lr + LPR * j;
            swv[j] = swr[min(c, nch - 1) / CPG];
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < M) {
            const float a = group_sum_f32<LPR>(acc[t]);
            if (lr == 0 && n < N)
                y[(int64_t)t * N + n] = f2h(a * (xsv[t] * 0.0625f));
        }
    }
}

template <int MT, int GS>
void launch_few_w4_m(const int8_t *xq, const float *xs, const uint8_t *w, const float *sw,
                     uint16_t *y, int M, int N, int K, hipStream_t st)
{
    const unsigned blocks = (unsigned)((N + 15) / 16);
    const size_t lds = (size_t)M * K;
    const int nch = K / 32;
    if (nch <= 64)
        hipLaunchKernelGGL((few_w4_kernel<MT, GS, 4>), dim3(blocks), dim3(256), lds, st, xq, xs, w,
                           sw, y, M, N, K);
    else if (nch <= 128)
        hipLaunchKernelGGL((few_w4_kernel<MT, GS, 8>), dim3(blocks), dim3(256), lds, st, xq, xs, w,
                           sw, y, M, N, K);
    else
        hipLaunchKernelGGL((few_w4_kernel<MT, GS, 16>), dim3(blocks), dim3(256), lds, st, xq, xs,
                           w, sw, y, M, N, K);
}

template <int GS>
void launch_few_w4_gs(const int8_t *xq, const float *xs, const uint8_t *w, const float *sw,
                      uint16_t *y, int M, int N, int K, hipStream_t st)
{
    if (M <= 1)
        launch_few_w4_m<1, GS>(xq, xs, w, sw, y, M, N, K, st);
    else if (M <= 2)
        launch_few_w4_m<2, GS>(xq, xs, w, sw, y, M, N, K, st);
    else
        launch_few_w4_m<4, GS>(xq, xs, w, sw, y, M, N, K, st);
}

template <int MT>
void launch_few_m(const int8_t *xq, const float *xs, const int8_t *w, const float *sw, uint16_t *y,
                  int M, int N, int K, hipStream_t st)
{
    const int nch = K / 16;
    if (nch <= 16 * 4)
        launch_few<MT, 16, 4>(xq, xs, w, sw, y, M, N, K, st);
    else if (nch <= 16 * 8)
        launch_few<MT, 16, 8>(xq, xs, w, sw, y, M, N, K, st);
    else if (nch <= 16 * 10)
        launch_few<MT, 16, 10>(xq, xs, w, sw, y, M, N, K, st);
    else if (nch <= 16 * 16)
        launch_few<MT, 16, 16>(xq, xs, w, sw, y, M, N, K, st);
    else
        launch_few<MT, 64, 16>(xq, xs, w, sw, y, M, N, K, st);
}

}  // namespace

void launch_few_pc(const int8_t *xq, const float *xs, const int8_t *w, const float *sw,
                   uint16_t *y, int M, int N, int K, hipStream_t st)
{
    if (M <= 1)
        launch_few_m<1>(xq, xs, w, sw, y, M, N, K, st);
    else if (M <= 2)
        launch_few_m<2>(xq, xs, w, sw, y, M, N, K, st);
    else
        launch_few_m<4>(xq, xs, w, sw, y, M, N, K, st);
}

void launch_few_w4(const int8_t *xq, const float *xs, const uint8_t *w, const float *sw, int gs,
                   uint16_t *y, int M, int N, int K, hipStream_t st)
{
    if (gs == 64)
        launch_few_w4_gs<64>(xq, xs, w, sw, y, M, N, K, st);
    else
        launch_few_w4_gs<128>(xq, xs, w, sw, y, M, N, K, st);
}

void launch_mv_group(bool int4, int gs, const uint16_t *x, const uint8_t *w, const float *sw,
                     uint16_t *y, int N, int K, int num_cu, hipStream_t st)
{
    const int cu = num_cu > 0 ? num_cu : 1;
    if (int4)
        (gs == 64 ? launch_group_k<true, 64> : launch_group_k<true, 128>)(x, w, sw, y, N, K, cu, st);
    else
        (gs == 64 ? launch_group_k<false, 64> : launch_group_k<false, 128>)(x, w, sw, y, N, K, cu, st);
}

}  // namespace w4a8
