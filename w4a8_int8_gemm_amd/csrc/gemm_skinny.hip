// Per-channel int8 GEMM for few tokens (up to 128): the weights streamed
// once (gfx950).
//
// Steps 3-4 of the kernel pipeline in the Apple-silicon essay ("Apple Silicon의
// AI 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계"):
// int32 accumulation of the int8 products, then the rescale by the token's and
// the output channel's scales.  With few tokens the layer is bound by reading
// the weights once (in the "cider" post's latency table for N=10240, K=2560
// the M = 128 row takes little more than the M = 1 row, one pass over the
// weights), so this form is built around keeping weight bytes in flight:
//
//  * Each workgroup owns a contiguous range of weight rows (a multiple of 8
//    rows; the ranges of all workgroups differ by at most 8 rows) and all M
//    tokens, so each weight byte is read from HBM once, by one compute unit.
//    The ranges are walked in passes of RB blocks of 16 rows.
//  * The four waves split K: wave w takes the 64-byte stages w, w + 4, ...
//    (rotated by a per-workgroup offset) of every row of the pass, so the two
//    halves of a 128-byte line go to two waves at the same time.  A wave copies
//    its own stages into its own LDS slots (buffer loads with the lds
//    modifier: four consecutive lanes fetch one row's 64 bytes, the access
//    pattern the memory pipeline coalesces) D stages ahead of the one it
//    computes, and reads its MFMA fragments back from there.  No other wave
//    touches those slots, so the main loop has no barriers: a wave only
//    waits for its own copies.
//  * v_mfma_i32_16x16x64_i8 with the weights as the first operand: lane l
//    supplies row l % 16 and 16-byte segment g' of the 64-byte stage of both
//    operands, g' = 0, 3, 1, 2 for l / 16 = 0 .. 3 (the same k for both,
//    which is all the product needs), and receives token l % 16 of rows
//    4 (l / 16) .. + 3 of the block.  In LDS a stage's 16-row block is 1 KiB,
//    64 bytes a row, with segment s of row r at s ^ ((r >> 2) & 3).  A
//    16-byte LDS read serves 16 lanes a cycle: per half-wave, those whose
//    4-lane quad index (lane bits 2-4) has one parity, as the LDS
//    bank-conflict counter shows -- rows 0-3 and 12-15 of one lane group and
//    rows 4-11 of the next.  Segments that differ by 3 between those two
//    groups put the 16 reads in distinct banks.
//  * At the end of a pass the four waves' int32 partial sums meet in LDS
//    (exact integer adds); each wave finishes a quarter of the blocks with the
//    same rescale as the tiled GEMM, so the fp16 outputs equal the tiled
//    GEMM's bit for bit (and the int32 export writes the sums).
//  * Rows past the range's end and tokens past M read as zeros (buffer
//    resources sized to the valid bytes); so do the stages past a wave's last
//    one (their offsets are moved past every buffer's end).  K % 64 == 0.
#include "kernels.hpp"
#include "lds_copy.hpp"

namespace w4a8 {

namespace {

constexpr int SKW = 4;                 // waves per workgroup
constexpr int SKU = 64;                // K bytes per stage (one MFMA depth)

template <int MB, int RB, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_skinny_kernel(GemmArgs args, int units, int i32_out)
{
    constexpr int NB = MB + RB;                       // 1 KiB blocks of a stage: X, then W
    constexpr int STAGE = NB * 1024;
    constexpr int WAVE_LDS = D * STAGE;
    constexpr int STAGING = SKW * WAVE_LDS;
    constexpr int RED = SKW * RB * MB * 1024;         // the waves' partial sums
    static_assert((D - 1) * NB < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) int8_t lds[STAGING > RED ? STAGING : RED];

    const int M = args.M, N = args.N, K = args.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int G = (int)gridDim.x, g = (int)blockIdx.x;
    // rows [r_begin, r_end): units of 8 rows split as evenly as possible
    const int u0 = (int)((int64_t)units * g / G), u1 = (int)((int64_t)units * (g + 1) / G);
    const int r_begin = 8 * u0, r_end = min(N, 8 * u1);
    // K in 64-byte units; wave w computes units w, w + 4, ..., so the two
    // halves of each 128-byte line are fetched by two waves at the same time
    const int nunit = K / SKU;
    const int nt = wave < nunit ? (nunit - 1 - wave) / SKW + 1 : 0;     // this wave's stages
    // Every workgroup reads all of X: the workgroups of an XCD (blockIdx
    // % 8) start at different units (a multiple of 4 apart, which keeps the
    // pairs), so that they do not all ask the same L2 lines at once
    const int rot = (SKW * (g >> 3)) % nunit;

    // copies: lane l fetches row l/4 of a block into physical segment l%4,
    // i.e. the logical segment the swizzle puts there (an involution)
    const int crow = lane >> 2;
    const uint32_t co = (uint32_t)(crow * K + 16 * ((lane & 3) ^ ((crow >> 2) & 3)));
    // fragments: lane l reads row l%16, logical segment g' (l/16 = g: 0, 3, 1, 2)
    const int frow = lane & 15;
    const int fseg = (3 * ((lane >> 4) & 1)) ^ (lane >> 5);
    const int fo = frow * 64 + 16 * (fseg ^ ((frow >> 2) & 3));
    const v4i rx = make_rsrc(args.xq, (uint32_t)(M * K));
    int8_t *const wl = lds + wave * WAVE_LDS;

    for (int p0 = r_begin; p0 < r_end; p0 += 16 * RB) {
        const int prow = min(16 * RB, r_end - p0);
        const v4i rw = make_rsrc(static_cast<const int8_t *>(args.w) + (int64_t)p0 * K,
                                 (uint32_t)(prow * K));
        if (p0 != r_begin)
            lds_barrier();                            // the previous pass is done with LDS

        v4i acc[RB][MB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[rb][mb] = v4i{0, 0, 0, 0};

        // The scales of the blocks this wave finishes (blocks wave, wave + 4,
        // ...), loaded before the pass's copies so that they arrive with the
        // first stage instead of costing a round trip at the end.  Indices
        // are clamped to the arrays; the int32 export has no scales and reads
        // (and ignores) the leading bytes of its operands instead.
        constexpr int NBW = (RB * MB + SKW - 1) / SKW;
        const float *const sa_src = i32_out ? reinterpret_cast<const float *>(args.xq) : args.sa;
        const float *const sw_src = i32_out ? static_cast<const float *>(args.w) : args.sw;
        float sa_pre[NBW], sw_pre[NBW][4];
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = min(wave + SKW * i, RB * MB - 1);
            const int rb = b / MB, mb = b % MB;
            const int m = mb * 16 + (lane & 15);
            const int n = p0 + rb * 16 + 4 * (lane >> 4);
            sa_pre[i] = sa_src[i32_out ? 0 : min(m, M - 1)];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sw_pre[i][r] = sw_src[i32_out ? 0 : min(n + r, N - 1)];
        }
        __builtin_amdgcn_sched_barrier(0);

        // Stage t of this wave (unit wave + 4 t, rotated) into slot d.
        auto copy = [&](int d, int t) __attribute__((always_inline)) {
            int u = wave + SKW * t + rot;
            u = u >= nunit ? u - nunit : u;
            const int k = u * SKU;
            const bool live = t < nt;
            const uint32_t oob = live ? 0u : 0x40000000u;
            const uint32_t kk = live ? (uint32_t)k : 0u;
            int8_t *sb = wl + d * STAGE;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                set_m0(lds_addr(sb + mb * 1024));
                copy16_buf_to_lds<0>(rx, co + (uint32_t)(mb * 16 * K) + oob, kk);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                set_m0(lds_addr(sb + (MB + rb) * 1024));
                copy16_buf_to_lds<0>(rw, co + (uint32_t)(rb * 16 * K) + oob, kk);
            }
        };
        auto compute = [&](int d) __attribute__((always_inline)) {
            const int8_t *sb = wl + d * STAGE + fo;
            v4i xa[MB], wa[RB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xa[mb] = *reinterpret_cast<const v4i *>(sb + mb * 1024);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                wa[rb] = *reinterpret_cast<const v4i *>(sb + (MB + rb) * 1024);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[rb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[rb], xa[mb], acc[rb][mb],
                                                                        0, 0, 0);
        };

        // stages 0 .. D-2 ahead; each step copies the stage D-1 ahead into the
        // slot the previous step consumed (its fragment reads are done: the
        // MFMAs that used them have issued), waits for its own stage and
        // computes it; the last nt % D stages are computed after the loop
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            copy(d, d);
        int t = 0;
        for (; t + D <= nt; t += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                __builtin_amdgcn_sched_barrier(0);
                copy((d + D - 1) % D, t + d + D - 1);
                wait_vmcnt<(D - 1) * NB>();
                __builtin_amdgcn_sched_barrier(0);
                compute(d);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();                              // every copy landed (none may write later)
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (t + d < nt)
                compute(d);

        // the four waves' sums meet in LDS; wave w finishes blocks b % 4 == w
        lds_barrier();                                // every wave is done with its slots
        v4i *red = reinterpret_cast<v4i *>(lds);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                red[((wave * RB + rb) * MB + mb) * 64 + lane] = acc[rb][mb];
        lds_barrier();
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wave + SKW * i;
            if (b >= RB * MB)
                break;
            const int rb = b / MB, mb = b % MB;
            v4i s = red[b * 64 + lane];
#pragma unroll
            for (int w = 1; w < SKW; ++w) {
                const v4i u = red[(w * RB * MB + b) * 64 + lane];
                s = v4i{s[0] + u[0], s[1] + u[1], s[2] + u[2], s[3] + u[3]};
            }
            const int m = mb * 16 + (lane & 15);
            const int n = p0 + rb * 16 + 4 * (lane >> 4);        // a multiple of 4
            if (m >= M || n >= r_end)
                continue;
            const bool whole = n + 3 < r_end;
            if (i32_out) {
                int32_t *C = static_cast<int32_t *>(args.out) + (int64_t)m * N + n;
                if (whole && (N & 3) == 0 && ((uintptr_t)args.out & 15) == 0) {
                    *reinterpret_cast<v4i *>(C) = s;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < r_end)
                            C[r] = s[r];
                }
            } else {
                uint16_t *Y = static_cast<uint16_t *>(args.out) + (int64_t)m * N + n;
                const float sam = sa_pre[i];
                uint16_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (n + r < r_end) ? f2h(rescale_pc(s[r], sam, sw_pre[i][r])) : (uint16_t)0;
                if (whole && (N & 3) == 0 && ((uintptr_t)args.out & 7) == 0) {
                    *reinterpret_cast<uint2 *>(Y) =
                        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                   (uint32_t)h[2] | ((uint32_t)h[3] << 16));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < r_end)
                            Y[r] = h[r];
                }
            }
        }
    }
}

// The blocks of 16 rows a pass covers: the fewest of the instantiated counts
// that hold the largest range, else the most (several passes).  The partial
// sums of four waves must fit LDS: RB x MB <= 32.
constexpr int skinny_max_rb(int mb) { return mb >= 8 ? 4 : 8; }
int skinny_rb(int mb, int rows)
{
    const int need = (rows + 15) / 16;
    for (int rb : {1, 2, 3, 4, 6, 8})
        if (rb >= need && rb <= skinny_max_rb(mb))
            return rb;
    return skinny_max_rb(mb);
}

int skinny_mb(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }

template <int MB, int RB>
void launch_skinny_t(const GemmArgs &a, int grid, int units, bool i32, hipStream_t st)
{
    // stages in flight per wave: as many as about 40 KiB of LDS per wave
    // holds, at most 4
    constexpr int NB = MB + RB;
    constexpr int D = NB <= 8 ? 4 : NB <= 13 ? 3 : 2;
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, RB, D>), dim3((unsigned)grid), dim3(64 * SKW), 0, st,
                       a, units, i32 ? 1 : 0);
}

template <int MB>
void launch_skinny_mb(int rb, const GemmArgs &a, int grid, int units, bool i32, hipStream_t st)
{
    switch (rb) {
    case 1: launch_skinny_t<MB, 1>(a, grid, units, i32, st); break;
    case 2: launch_skinny_t<MB, 2>(a, grid, units, i32, st); break;
    case 3: launch_skinny_t<MB, 3>(a, grid, units, i32, st); break;
    case 4: launch_skinny_t<MB, 4>(a, grid, units, i32, st); break;
    default:
        if constexpr (skinny_max_rb(MB) >= 8) {
            if (rb == 6)
                launch_skinny_t<MB, 6>(a, grid, units, i32, st);
            else
                launch_skinny_t<MB, 8>(a, grid, units, i32, st);
        }
        break;
    }
}

}  // namespace

TileInfo launch_gemm_skinny(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch)
{
    const int units = (a.N + 7) / 8;
    const int cu = a.num_cu > 0 ? a.num_cu : 1;
    const int grid = units < cu ? units : cu;
    const int rows = 8 * ((units + grid - 1) / grid);
    const int mb = skinny_mb(a.M);
    const int rb = skinny_rb(mb, rows);
    if (launch) {
        switch (mb) {
        case 1: launch_skinny_mb<1>(rb, a, grid, units, i32_out, st); break;
        case 2: launch_skinny_mb<2>(rb, a, grid, units, i32_out, st); break;
        case 4: launch_skinny_mb<4>(rb, a, grid, units, i32_out, st); break;
        default: launch_skinny_mb<8>(rb, a, grid, units, i32_out, st); break;
        }
    }
    TileInfo r{};
    r.bm = 16 * mb;
    r.bn = 16 * rb;
    r.waves = SKW;
    r.tiles = grid;
    r.grid = grid;
    r.per_cu = 1;
    return r;
}

}  // namespace w4a8
