// Per-channel int8 GEMM for a few dozen to a few hundred tokens: the weights
// streamed once, the activations shared through LDS (gfx950).
//
// Steps 3-4 of the kernel pipeline in the Apple-silicon essay ("Apple Silicon의
// AI 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계"):
// int32 accumulation of the int8 products, then the rescale by the token's and
// the output channel's scales.  Between one token and a full prefill the layer
// is bound by moving bytes, not by the matrix cores (the "cider" post's latency
// table for N=10240, K=2560 has the M = 128 row close to the M = 1 row): the
// weights must come from HBM once, and every compute unit needs the
// activations of the tokens it serves.  So:
//
//  * The grid is one workgroup per compute unit.  Workgroup g owns a
//    contiguous range of weight rows (units of 8 rows, ranges within 8 rows of
//    each other) and one of PM slices of the tokens (PM = 1 or 2, the split
//    that moves the fewest bytes per compute unit); the PM workgroups of one
//    row range sit on one XCD (one L2), so the weights still come from HBM
//    once.
//  * K advances in stages of 128 bytes -- whole 128-byte lines of every row
//    -- through a ring of D stages in LDS (D = 4 to 8: as many as about
//    144 KiB hold), copied from global memory straight into LDS.  The four
//    waves share every stage: each copies a quarter of its 1 KiB blocks (8 rows
//    of 128 bytes), and one barrier per stage publishes it.  With D - 3 later
//    stages in flight, a compute unit keeps 50-100 KiB of loads outstanding,
//    which the HBM latency needs.  A stage's fragments are read from LDS one
//    iteration ahead, beside the MFMAs of the stage before.
//  * The waves split the tokens (MBW blocks of 16 each) and take all rows
//    (RB blocks of 16): v_mfma_i32_16x16x64_i8 with the weights as the first
//    operand, two k-steps per stage.  A lane of the result holds one token and
//    four consecutive rows, the output's 8-byte runs.
//  * Chunk c of LDS row r sits at c ^ (r & 7) ^ ((r >> 3) & 1).  A 16-byte LDS
//    read serves 16 lanes a cycle: per half-wave, those whose 4-lane quad
//    index (lane bits 2-4) has one parity, as the LDS bank-conflict counter
//    shows -- rows 0-3 and 12-15 of a fragment from one lane group and rows
//    4-11 from the next.  Lanes 0-15, 16-31, 32-47, 48-63 take the k chunks
//    4h, 4h + 2, 4h + 1, 4h + 3 of k-step h (any order serves the product if
//    both operands use it): two chunks 2 apart put those 16 reads in distinct
//    banks, where chunks 1 apart would meet in half of them.
//  * The row ranges of an XCD start their K loop at different stages (the sum
//    is exact in any order), so that its compute units do not all ask for the
//    same lines of the activations at once; the token slices of one range
//    start at the same stage, so the weights stay a single HBM stream.
//  * Rows past the range, tokens past the slice and stages past the end read
//    as zeros (buffer resources sized to the valid bytes).  K % 128 == 0.
//  * The epilogue is the tiled GEMM's rescale, so the fp16 outputs equal the
//    tiled GEMM's bit for bit (and the int32 export writes the sums).
#include "kernels.hpp"
#include "lds_copy.hpp"

namespace w4a8 {

namespace {

constexpr int RWW = 4;                 // waves per workgroup
constexpr int RSK = 128;               // K bytes per stage

__device__ __forceinline__ int rswz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// MBW: token blocks of 16 per wave; RB: row blocks of 16 per workgroup;
// D: ring depth.
template <int MBW, int RB, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_rows_kernel(GemmArgs args, int units, int pm_slices, int i32_out)
{
    constexpr int XR = RWW * 16 * MBW;                // token rows of a stage
    constexpr int RBP = (RB + 1) & ~1;                // row blocks copied (even: the
    constexpr int WR = 16 * RBP;                      //   blocks split over the waves)
    constexpr int NBLK = (XR + WR) / 8;               // 1 KiB blocks per stage
    static_assert(NBLK % RWW == 0, "stage blocks must split evenly over the waves");
    constexpr int NCW = NBLK / RWW;                   // copies per wave per stage
    constexpr int STAGE = NBLK * 1024;
    static_assert((D - 2) * NCW < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) int8_t ring[D * STAGE];

    const int M = args.M, N = args.N, K = args.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int G = (int)gridDim.x, g = (int)blockIdx.x;

    // ---- this workgroup's tokens and rows.  Workgroups are dealt to the 8
    // XCDs round robin (g % 8); the pm_slices workgroups of one row range are
    // consecutive within an XCD.
    const int xcd = g & 7, local = g >> 3, per_xcd = G >> 3;
    const int pm = local % pm_slices;
    const int ranges = G / pm_slices;
    const int pn = xcd * (per_xcd / pm_slices) + local / pm_slices;
    const int u0 = (int)((int64_t)units * pn / ranges);
    const int u1 = (int)((int64_t)units * (pn + 1) / ranges);
    const int r_begin = 8 * u0, r_end = min(N, 8 * u1);
    const int m_slice = (M + pm_slices - 1) / pm_slices;
    const int m_begin = pm * m_slice, m_end = min(M, m_begin + m_slice);
    const int nstage = K / RSK;
    // K start: row ranges of an XCD a multiple of 4 stages apart; the token
    // slices of one range start together, so the second asks for the same
    // weight lines as the first while they are still in L2
    const int rot = (4 * (local / pm_slices)) % nstage;

    const v4i rx = make_rsrc(args.xq + (int64_t)m_begin * K,
                             (uint32_t)(max(0, m_end - m_begin) * K));
    const v4i rw = make_rsrc(static_cast<const int8_t *>(args.w) + (int64_t)r_begin * K,
                             (uint32_t)(max(0, r_end - r_begin) * K));

    // ---- copies.  Block b of a stage holds rows 8b .. 8b+7 of the stage
    // (tokens first, then weight rows); lane l writes LDS row 8b + l/8, physical
    // chunk l%8, so it fetches the logical chunk the swizzle puts there.  Wave w
    // copies blocks w, w + 4, ...
    uint32_t voff[NCW];
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
        const int b = wave + RWW * i;
        const int row = (b < XR / 8 ? b : b - XR / 8) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3) ^ (b & 1);
        voff[i] = (uint32_t)(row * K + 16 * c);
    }
    auto issue_stage = [&](int slot, int t) __attribute__((always_inline)) {
        // stage t of this workgroup's stream (t >= nstage: no stage, read zeros)
        int st = t + rot;
        st = st >= nstage ? st - nstage : st;
        const bool live = t < nstage;
        const uint32_t kk = live ? (uint32_t)(st * RSK) : 0u;
        const uint32_t oob = live ? 0u : 0x40000000u;
        int8_t *base = ring + slot * STAGE;
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            const int b = wave + RWW * i;
            set_m0(lds_addr(base + b * 1024));
            copy16_buf_to_lds<0>(b < XR / 8 ? rx : rw, voff[i] + oob, kk);
        }
    };

    // ---- fragments: lane l reads row l%16 of a 16-row block, logical chunk
    // 4h + g for k-step h, g = 0, 2, 1, 3 for lane groups l/16 = 0 .. 3
    // (blocks start at multiples of 16 rows)
    const int frow = lane & 15;
    const int fg = (((lane >> 4) & 1) << 1) | (lane >> 5);
    int fo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        fo[h] = frow * RSK + 16 * rswz(frow, 4 * h + fg);

    v4i acc[RB][MBW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            acc[rb][mb] = v4i{0, 0, 0, 0};

    // the fragments of one stage: both k-steps, tokens then rows
    struct Frag {
        v4i x[2][MBW], w[2][RB];
    };
    auto read_frags = [&](Frag &F, int slot) __attribute__((always_inline)) {
        const int8_t *base = ring + slot * STAGE;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                F.x[h][mb] =
                    *reinterpret_cast<const v4i *>(base + ((wave * MBW + mb) * 16) * RSK + fo[h]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                F.w[h][rb] = *reinterpret_cast<const v4i *>(base + (XR + rb * 16) * RSK + fo[h]);
        }
    };
    auto compute = [&](const Frag &F) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
                    acc[rb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(F.w[h][rb], F.x[h][mb],
                                                                        acc[rb][mb], 0, 0, 0);
    };

    // ---- pipeline.  Stages 0 .. D-2 are issued up front and stage 0's
    // fragments read.  Iteration s waits for its own copies of stage s+1 (the
    // D-3 later stages stay in flight), barriers -- stage s+1 is visible and
    // every wave is done with stage s-1, whose fragments it read an iteration
    // earlier -- issues stage s+D-1 into the slot stage s-1 vacated, reads
    // stage s+1's fragments and computes stage s from the fragments read in
    // the previous iteration, so the LDS reads run beside the MFMAs.
    static_assert(D >= 3, "ring depth");
    // The epilogue's scales are loaded first, so that they arrive with the
    // first stage instead of costing a round trip after the last one.
    // Indices are clamped to the arrays; the int32 export has no scales and
    // reads (and ignores) the leading bytes of its operands instead.
    const float *const sa_src = i32_out ? reinterpret_cast<const float *>(args.xq) : args.sa;
    const float *const sw_src = i32_out ? static_cast<const float *>(args.w) : args.sw;
    float sa_pre[MBW], sw_pre[RB][4];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int m = m_begin + (wave * MBW + mb) * 16 + (lane & 15);
        sa_pre[mb] = sa_src[i32_out ? 0 : min(m, M - 1)];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = r_begin + rb * 16 + 4 * (lane >> 4) + r;
            sw_pre[rb][r] = sw_src[i32_out ? 0 : min(n, N - 1)];
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < D - 1; ++t)
        issue_stage(t, t);
    Frag f0, f1;
    wait_vmcnt<(D - 2) * NCW>();
    lds_barrier();
    read_frags(f0, 0);
    int slot = 0;                                     // slot of stage s
    auto iteration = [&](int s, Frag &cur, Frag &nxt) __attribute__((always_inline)) {
        const int nslot = slot == D - 1 ? 0 : slot + 1;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(D - 3) * NCW>();
        lds_barrier();
        issue_stage(slot == 0 ? D - 1 : slot - 1, s + D - 1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(nxt, nslot);                       // past the last stage: zeros, unused
        compute(cur);
        slot = nslot;
    };
    int s = 0;
    for (; s + 2 <= nstage; s += 2) {
        iteration(s, f0, f1);
        iteration(s + 1, f1, f0);
    }
    if (s < nstage)
        iteration(s, f0, f1);
    // no copy may still be writing LDS when the workgroup ends
    wait_vmcnt<0>();

    // ---- outputs: lane l holds token (wave MBW + mb) 16 + l%16 of the slice
    // and rows rb 16 + 4 (l/16) + 0..3 of the range
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int m = m_begin + (wave * MBW + mb) * 16 + (lane & 15);
        if (m >= m_end)
            continue;
        const float sam = sa_pre[mb];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int n = r_begin + rb * 16 + 4 * (lane >> 4);
            if (n >= r_end)
                continue;
            const v4i s = acc[rb][mb];
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
                uint16_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (n + r < r_end) ? f2h(rescale_pc(s[r], sam, sw_pre[rb][r])) : (uint16_t)0;
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

// Ring depth: as many stages as about 144 KiB hold, at most 8.
constexpr int rows_depth(int mbw, int rb)
{
    const int stage = (RWW * 16 * mbw + 16 * ((rb + 1) & ~1)) * RSK;
    const int d = (144 * 1024) / stage;
    return d > 8 ? 8 : d;
}

template <int MBW, int RB>
void launch_rows_t(const GemmArgs &a, int grid, int units, int pm, bool i32, hipStream_t st)
{
    constexpr int D = rows_depth(MBW, RB);
    static_assert(D >= 3, "ring depth");
    hipLaunchKernelGGL((gemm_rows_kernel<MBW, RB, D>), dim3((unsigned)grid), dim3(64 * RWW), 0, st,
                       a, units, pm, i32 ? 1 : 0);
}

template <int MBW>
void launch_rows_mbw(int rb, const GemmArgs &a, int grid, int units, int pm, bool i32,
                     hipStream_t st)
{
    switch (rb) {
    case 1: launch_rows_t<MBW, 1>(a, grid, units, pm, i32, st); break;
    case 2: launch_rows_t<MBW, 2>(a, grid, units, pm, i32, st); break;
    case 3: launch_rows_t<MBW, 3>(a, grid, units, pm, i32, st); break;
    case 4: launch_rows_t<MBW, 4>(a, grid, units, pm, i32, st); break;
    case 5: launch_rows_t<MBW, 5>(a, grid, units, pm, i32, st); break;
    case 6: launch_rows_t<MBW, 6>(a, grid, units, pm, i32, st); break;
    case 7: launch_rows_t<MBW, 7>(a, grid, units, pm, i32, st); break;
    default: launch_rows_t<MBW, 8>(a, grid, units, pm, i32, st); break;
    }
}

}  // namespace

RowsPlan plan_gemm_rows(int M, int N, int K, int num_cu)
{
    RowsPlan p{};
    p.ok = false;
    // one workgroup per compute unit, a multiple of 8 (one per XCD slot)
    const int grid = (num_cu / 8) * 8;
    if (grid < 8 || K < RSK || K % RSK != 0 || M < 1 || N < 1)
        return p;
    const int units = (N + 7) / 8;
    int best = 0;
    for (int pm : {1, 2}) {
        const int ranges = grid / pm;
        if ((grid / 8) % pm != 0)
            continue;
        const int m_slice = (M + pm - 1) / pm;
        const int mbw = (m_slice + 63) / 64;          // token blocks of 16 per wave
        const int rows = 8 * ((units + ranges - 1) / ranges);
        const int rb = (rows + 15) / 16;
        if (mbw > 2 || rb > 8)
            continue;
        // bytes a compute unit copies per stage, padded as the kernel pads them
        const int cost = 64 * mbw + 16 * ((rb + 1) & ~1);
        if (best == 0 || cost < best) {
            best = cost;
            p.ok = true;
            p.pm = pm;
            p.mbw = mbw;
            p.rb = rb;
            p.grid = grid;
            p.units = units;
        }
    }
    return p;
}

TileInfo launch_gemm_rows(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch)
{
    const RowsPlan p = plan_gemm_rows(a.M, a.N, a.K, a.num_cu);
    if (launch && p.ok) {
        if (p.mbw == 1)
            launch_rows_mbw<1>(p.rb, a, p.grid, p.units, p.pm, i32_out, st);
        else
            launch_rows_mbw<2>(p.rb, a, p.grid, p.units, p.pm, i32_out, st);
    }
    TileInfo r{};
    r.bm = p.ok ? RWW * 16 * p.mbw : 0;
    r.bn = p.ok ? 16 * p.rb : 0;
    r.waves = RWW;
    r.tiles = p.ok ? p.grid : 0;
    r.grid = p.ok ? p.grid : 0;
    r.per_cu = 1;
    return r;
}

}  // namespace w4a8
