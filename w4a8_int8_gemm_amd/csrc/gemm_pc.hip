// Per-channel int8 GEMM for large outputs on 256 x 320 tiles (gfx950).
//
// Steps 3-4 of the kernel pipeline in the Apple-silicon essay ("Apple Silicon의
// AI 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계"): the
// INT8 GEMM accumulates in INT32, then each sum is rescaled by the product of
// its token's and its output channel's scales to FP16.
//
// Why a second kernel: at the matrix cores' rate a 256 x 160 tile per compute
// unit pulls about 42 bytes per cycle from L2 into LDS, close to what a
// compute unit's share of its L2 delivers, and the waves of such a kernel
// spend much of their time waiting for those copies.  A 256 x 320 tile needs
// 31 % fewer bytes per multiply-add (29 bytes per cycle).  Its accumulators
// do not fit four waves, so eight waves (two per SIMD) compute 64 x 160 each.
//
//  * Waves: wave w covers rows 64 (w % 4) .. + 63 and columns 160 (w / 4) ..
//    + 159 of the tile: 2 x 5 blocks of v_mfma_i32_32x32x32_i8 with the
//    weights as the first operand (a lane holds one output row and runs of
//    four columns, which the epilogue stores as they are).
//  * K advances in stages of 128 bytes -- whole 128-byte lines of each row;
//    half-line stages cost more in the memory pipeline than they save -- through
//    two LDS buffers of 72 KiB: 32 blocks of 1 KiB (8 rows) of X and 40 of W,
//    copied from global memory straight into LDS (buffer loads with the lds
//    modifier).  Only waves 0-3 copy (8 X blocks and 10 W blocks each per
//    stage), so the other wave on each SIMD is a pure stream of MFMAs and
//    fragment reads that keeps the matrix core busy while its sibling's
//    instruction stream waits on the memory pipeline (a uniform split of the
//    copies over all eight waves ran 8 % slower).  Chunk c of row r sits at
//    c ^ (r & 7) ^ ((r >> 3) & 1): the 16 rows one LDS read cycle serves (one
//    logical chunk each) hit distinct banks.
//  * Iteration u computes stage u in four k-steps, each reading the next
//    step's fragments while it runs.  After step 2 every wave has read all of
//    stage u, so a wait for stage u+1 and a barrier come there; step 3 reads
//    the first fragments of stage u+1 and issues the copies of stage u+2 into
//    the buffer stage u vacated, which gives them four k-steps to land.
//  * Persistent: each workgroup walks a list of tiles in an order that keeps
//    the tiles in flight on one XCD (one L2) on shared rows of X and W; its
//    stages form one stream across its tiles.
//  * Rows past the end of X or W read as zeros (per-tile buffer resources).
#include "kernels.hpp"
#include "lds_copy.hpp"

namespace w4a8 {

namespace {

constexpr int QBM = 256, QBN = 320;            // output tile per workgroup
constexpr int QBK = 128;                       // k bytes per stage: four 32-wide MFMA steps
constexpr int QNW = 8;                         // waves: 4 (m) x 2 (n)
constexpr int QXB = QBM * QBK, QWB = QBN * QBK;
constexpr int QSB = QXB + QWB;                 // 72 KiB per stage; two stages
constexpr int QCW = 4;                         // copying waves (0 .. 3, one per SIMD)
constexpr int QXC = QXB / 1024 / QCW;          // X blocks per copying wave per stage (8)
constexpr int QWC = QWB / 1024 / QCW;          // W blocks per copying wave per stage (10)
constexpr int QNC = QXC + QWC;                 // copies per copying wave per stage (18)
constexpr int QFM = 2, QFN = 5;                // 32 x 32 blocks per wave (m, n)
constexpr int QESN = QBM + QBN;                // epilogue scales of a tile
constexpr int QEW = (QESN + 64 * QNW - 1) / (64 * QNW);   // their copy instructions per wave (2)

typedef int v16i_t __attribute__((ext_vector_type(16)));

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row r (128 bytes).
__device__ __forceinline__ int swz128(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

template <bool I32OUT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pc2_kernel(GemmArgs args, int tiles_m, int tiles_n, int group_m)
{
    __shared__ __attribute__((aligned(1024))) int8_t ring[2 * QSB];
    __shared__ __attribute__((aligned(16))) float eps[QEW * QNW * 64];

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;

    // ---- this workgroup's tiles (XCD-contiguous renumbering, groups of
    // group_m tile rows)
    const int G = (int)gridDim.x;
    int wl;
    {
        const int bid = (int)blockIdx.x;
        const int xcd = bid & 7, local = bid >> 3;
        const int per = G >> 3, rem = G & 7;
        wl = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    }
    const int total = tiles_m * tiles_n;
    const int ntile = (total - wl + G - 1) / G;       // >= 1: the grid has at most `total` groups
    auto tile_origin = [&](int i, int &m0, int &n0) __attribute__((always_inline)) {
        const int lid = i * G + wl;
        const int span = group_m * tiles_n;
        const int first_m = (lid / span) * group_m;
        const int gm = min(tiles_m - first_m, group_m);
        const int in = lid % span;
        m0 = (first_m + in % gm) * QBM;
        n0 = (in / gm) * QBN;
    };
    const int nstage = K / QBK;                       // K % 128 == 0 on this kernel
    const int U = ntile * nstage;

    // ---- copies.  Lane l of a block copy writes LDS row l/8 of the block,
    // physical chunk l%8, so it fetches the logical chunk the swizzle puts
    // there (an involution): (l%8) ^ (row & 7) ^ ((row >> 3) & 1), with
    // row = 8 blk + l/8.  The lane's offset is 8 blk K plus a part that
    // depends on the block only through its parity (added per copy: the row
    // must be in the per-lane offset, which the buffer's range check covers,
    // unlike the scalar offset that carries the stage's k).
    uint32_t vo[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        vo[par] = (uint32_t)((lane >> 3) * K + 16 * ((lane & 7) ^ (lane >> 3) ^ par));

    struct Src {
        int v;         // stage in this workgroup's stream (clamped to U - 1)
        int s;         // stage within its tile
        int tile;      // tile within this workgroup's list
        int buf;       // LDS buffer (unclamped stage index mod 2)
        int m0, n0;
        v4i rx, rw;
    };
    auto set_tile = [&](Src &c, int i) __attribute__((always_inline)) {
        c.tile = i;
        tile_origin(i, c.m0, c.n0);
        c.rx = make_rsrc(args.xq + (int64_t)c.m0 * K, (uint32_t)(min(QBM, M - c.m0) * K));
        c.rw = make_rsrc(static_cast<const int8_t *>(args.w) + (int64_t)c.n0 * K,
                         (uint32_t)(min(QBN, N - c.n0) * K));
    };
    auto advance = [&](Src &c) __attribute__((always_inline)) {
        c.buf ^= 1;
        if (c.v + 1 < U) {                            // past the end: repeat the last stage
            ++c.v;
            if (++c.s == nstage) {
                c.s = 0;
                set_tile(c, c.tile + 1);
            }
        }
    };
    // Copy p (0 <= p < 18) of a stage by copying wave `wave`: its X blocks,
    // then its W blocks.
    auto issue_copy = [&](const Src &src, int p) __attribute__((always_inline)) {
        const uint32_t k0 = (uint32_t)(src.s * QBK);
        int8_t *base = ring + src.buf * QSB;
        const bool isx = p < QXC;
        const int blk = isx ? wave * QXC + p : wave * QWC + (p - QXC);
        const uint32_t voff = ((blk & 1) ? vo[1] : vo[0]) + (uint32_t)(blk * 8 * K);
        set_m0(lds_addr(base + (isx ? 0 : QXB) + blk * 1024));
        copy16_buf_to_lds<0>(isx ? src.rx : src.rw, voff, k0);
    };
    // The epilogue scales of the tile at (m0, n0): sa of its rows, then sw of
    // its columns (rows and columns past the end repeat the last one).
    auto issue_epilogue_scales = [&](int m0, int n0) __attribute__((always_inline)) {
        if constexpr (!I32OUT) {
#pragma unroll
            for (int i = 0; i < QEW; ++i) {
                const int e = (wave + QNW * i) * 64 + lane;
                const float *src;
                if (e < QBM)
                    src = args.sa + min(m0 + e, M - 1);
                else if (e < QESN)
                    src = args.sw + min(n0 + e - QBM, N - 1);
                else
                    src = args.sa + min(m0, M - 1);   // padding slot, never read
                copy4_to_lds(src, lds_addr(eps + (wave + QNW * i) * 64));
            }
        }
    };

    // ---- fragments: lane reads row base + l%32, logical chunk 2t + l/32 of
    // k-step t (bases are multiples of 32, so the swizzle depends on l%32)
    const int lrow = lane & 31, lhalf = lane >> 5;
    int fo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        fo[t] = lrow * QBK + swz128(lrow, 2 * t + lhalf) * 16;
    struct Frag {
        v4i a[QFN];    // weights (first operand)
        v4i b[QFM];    // activations
    };
    Frag f0, f1;
    // fragment r of k-step t from buffer buf, in the order the step's MFMAs
    // first use them: a0, b0, b1, a1, a2, a3, a4
    auto read_one = [&](Frag &F, int buf, int t, int r) __attribute__((always_inline)) {
        const int8_t *xb = ring + buf * QSB + wm * 64 * QBK + fo[t];
        const int8_t *wb = ring + buf * QSB + QXB + wn * 160 * QBK + fo[t];
        if (r == 0)
            F.a[0] = *reinterpret_cast<const v4i *>(wb);
        else if (r < 3)
            F.b[r - 1] = *reinterpret_cast<const v4i *>(xb + (r - 1) * 32 * QBK);
        else
            F.a[r - 2] = *reinterpret_cast<const v4i *>(wb + (r - 2) * 32 * QBK);
    };

    v16i_t acc[QFN][QFM];
#pragma unroll
    for (int j = 0; j < QFN; ++j)
#pragma unroll
        for (int i = 0; i < QFM; ++i)
            acc[j][i] = v16i_t{};

    // The ten MFMAs of one k-step on F (restarting the sums when RESTART),
    // with the seven fragment reads of the next step into G after MFMAs
    // 0, 0, 1, 2, 2, 3, 4, and (COPIES, copying waves only) the 18 copies of
    // the stage `src`, two after each of MFMAs 0 .. 8.
    const bool copier = wave < QCW;
    auto mfma_step = [&](const Frag &F, auto RESTART, Frag &G, int rbuf, int rt, const Src &src,
                         auto COPIES) __attribute__((always_inline)) {
        constexpr bool restart = decltype(RESTART)::value;
        constexpr bool copies = decltype(COPIES)::value;
#pragma unroll
        for (int k = 0; k < QFN * QFM; ++k) {
            const int j = k / QFM, i = k % QFM;
            acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.a[j], F.b[i],
                                                              restart ? v16i_t{} : acc[j][i], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 7; ++r)
                if ((r * 10) / 14 == k)
                    read_one(G, rbuf, rt, r);
            if (copies && k < QNC / 2 && copier) {
                issue_copy(src, 2 * k);
                issue_copy(src, 2 * k + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- the tile's outputs
    auto epilogue = [&](int m0, int n0) __attribute__((always_inline)) {
        const int lr = lane & 31, lh = lane >> 5;
        const int mw = m0 + wm * 64, nw = n0 + wn * 160;
        if constexpr (I32OUT) {
            // Lane l holds row mw + 32 i + l%32 of block (j, i) and columns
            // nw + 32 j + 8 g + 4 (l/32) + 0..3 in elements 4g..4g+3.
            int32_t *C = static_cast<int32_t *>(args.out);
#pragma unroll
            for (int j = 0; j < QFN; ++j)
#pragma unroll
                for (int i = 0; i < QFM; ++i) {
                    const int m = mw + 32 * i + lr;
                    if (m >= M)
                        continue;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = nw + 32 * j + 8 * g + 4 * lh;
                        if (n + 3 < N && (N & 3) == 0) {
                            *reinterpret_cast<v4i *>(C + (int64_t)m * N + n) =
                                v4i{acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2],
                                    acc[j][i][4 * g + 3]};
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < N)
                                    C[(int64_t)m * N + n + r] = acc[j][i][4 * g + r];
                        }
                    }
                }
        } else {
            uint16_t *Y = static_cast<uint16_t *>(args.out);
            float sam[QFM];                         // sa of this lane's rows
#pragma unroll
            for (int i = 0; i < QFM; ++i)
                sam[i] = eps[wm * 64 + i * 32 + lr];
            const float *swp = eps + QBM + wn * 160;
            // whole tile inside the output, rows a multiple of 16 bytes and a
            // 16-byte aligned output: every 16-byte store is in bounds and aligned
            const bool fast = m0 + QBM <= M && n0 + QBN <= N && (N & 7) == 0 &&
                              ((uintptr_t)Y & 15) == 0;
            if (fast) {
                const uint32_t voff = (uint32_t)((lr * N + 8 * lh) * 2);
#pragma unroll
                for (int j = 0; j < QFN; ++j) {
#pragma unroll
                    for (int i = 0; i < QFM; ++i) {
                        uint32_t d[8];
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            // sw of columns 32 j + 8 g + 4 lh + 0..3
                            const v4f swv =
                                *reinterpret_cast<const v4f *>(&swp[j * 32 + 8 * g + 4 * lh]);
                            float v[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                v[r] = rescale_pc(acc[j][i][4 * g + r], sam[i], swv[r]);
                            d[2 * g] = pack_h2(v[0], v[1]);
                            d[2 * g + 1] = pack_h2(v[2], v[3]);
                        }
                        // trade the upper lanes' group g with the lower lanes'
                        // group g + 1 (g even): lanes 0-31 then hold columns
                        // 16 (g/2) + 0..7, lanes 32-63 columns 16 (g/2) + 8..15
#pragma unroll
                        for (int g = 0; g < 4; g += 2)
#pragma unroll
                            for (int w = 0; w < 2; ++w)
                                lane_half_swap(d[2 * g + w], d[2 * g + 2 + w]);
                        char *blk = reinterpret_cast<char *>(Y + (int64_t)(mw + i * 32) * N + nw +
                                                             j * 32) + voff;
                        *reinterpret_cast<v4u *>(blk) = v4u{d[0], d[1], d[2], d[3]};
                        *reinterpret_cast<v4u *>(blk + 32) = v4u{d[4], d[5], d[6], d[7]};
                        // one 32 x 32 block at a time (keeps the live registers few)
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < QFN; ++j)
#pragma unroll
                    for (int i = 0; i < QFM; ++i) {
                        const int m = mw + i * 32 + lr;
                        if (m < M) {
#pragma unroll
                            for (int g = 0; g < 4; ++g)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int nl = j * 32 + 8 * g + 4 * lh + r;
                                    if (nw + nl < N)
                                        Y[(int64_t)m * N + nw + nl] =
                                            f2h(rescale_pc(acc[j][i][4 * g + r], sam[i], swp[nl]));
                                }
                        }
                    }
            }
        }
    };

    // ---- pipeline.  Stage u lives in buffer u & 1.  Iteration u: steps 0-2
    // compute stage u (each reading the next step's fragments, the last of
    // them stage u's step-3 fragments); wait for stage u+1 (issued in
    // iteration u-1, the only copies in flight) and barrier -- after it every
    // wave is done reading buffer u & 1; step 3 computes stage u's last
    // k-step, reads the first fragments of stage u+1 from the other buffer
    // and (waves 0-3) issues the copies of stage u+2 into buffer u & 1.  Past the
    // end of the stream the copies repeat the last stage into a buffer nobody
    // reads.  A tile's epilogue scales, copied after the previous tile's
    // epilogue, have landed at the next wait like everything else.
    Src cp;                                           // stage whose copies come next
    cp.v = 0; cp.s = 0; cp.buf = 0;
    set_tile(cp, 0);
    int cm0 = cp.m0, cn0 = cp.n0, ctile = 0;          // the tile being computed
    issue_epilogue_scales(cm0, cn0);
    if (copier) {
#pragma unroll
        for (int p = 0; p < QNC; ++p)                 // stage 0
            issue_copy(cp, p);
    }
    advance(cp);
    if (copier) {
#pragma unroll
        for (int p = 0; p < QNC; ++p)                 // stage 1
            issue_copy(cp, p);
        wait_vmcnt<QNC>();                            // stage 0 landed (stage 1 may not have)
    } else {
        wait_vmcnt<0>();                              // the epilogue scales
    }
    advance(cp);                                      // stage 2: issued in iteration 0
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 7; ++r)
        read_one(f0, 0, 0, r);

    int b = 0, s = 0;                                 // buffer and in-tile stage of iteration u
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (s == 0)
            mfma_step(f0, std::true_type(), f1, b, 1, cp, std::false_type());
        else
            mfma_step(f0, std::false_type(), f1, b, 1, cp, std::false_type());
        mfma_step(f1, std::false_type(), f0, b, 2, cp, std::false_type());
        mfma_step(f0, std::false_type(), f1, b, 3, cp, std::false_type());
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();
        lds_barrier();
        mfma_step(f1, std::false_type(), f0, b ^ 1, 0, cp, std::true_type());
        __builtin_amdgcn_sched_barrier(0);

        if (s + 1 == nstage) {                        // the tile is done
            epilogue(cm0, cn0);
            s = 0;
            if (++ctile < ntile) {
                tile_origin(ctile, cm0, cn0);
                if constexpr (!I32OUT) {
                    lds_barrier();                    // every wave is done with the scales
                    issue_epilogue_scales(cm0, cn0);
                }
            }
        } else {
            ++s;
        }
        advance(cp);
        b ^= 1;
    }
    // no copy may still be writing LDS when the workgroup ends
    wait_vmcnt<0>();
}

template <bool I32OUT>
int groups_per_cu_pc2()
{
    static const int occ = [] {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_pc2_kernel<I32OUT>, 512, 0) !=
                hipSuccess || o < 1)
            o = 1;
        return o;
    }();
    return occ;
}

template <bool I32OUT>
TileInfo launch_pc2_impl(const GemmArgs &a, hipStream_t st, bool launch)
{
    const int tiles_m = (a.M + QBM - 1) / QBM, tiles_n = (a.N + QBN - 1) / QBN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t resident = (int64_t)a.num_cu * groups_per_cu_pc2<I32OUT>();
    const int64_t grid = tiles < resident ? tiles : resident;
    if (launch)
        hipLaunchKernelGGL((gemm_pc2_kernel<I32OUT>), dim3((unsigned)grid), dim3(512), 0, st, a,
                           tiles_m, tiles_n, 4);
    TileInfo r{};
    r.bm = QBM; r.bn = QBN; r.waves = QNW;
    r.tiles = tiles;
    r.grid = grid;
    r.per_cu = groups_per_cu_pc2<I32OUT>();
    return r;
}

}  // namespace

TileInfo launch_gemm_pc2(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch)
{
    return i32_out ? launch_pc2_impl<true>(a, st, launch) : launch_pc2_impl<false>(a, st, launch);
}

}  // namespace w4a8
