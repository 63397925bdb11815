// int8 x int8 -> int32 GEMMs on gfx950 matrix cores, with their epilogues.
//
// Steps 3-4 of the kernel pipeline in the Apple-silicon essay ("Apple Silicon의
// AI 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계"): the
// INT8 GEMM accumulates in INT32 and the sums are rescaled by the product of
// activation and weight scales to FP16.  Per-group scales need the partial
// sums of each group rescaled during accumulation (same essay, section
// "입도: Per-Tensor vs. Per-Channel vs. Per-Group").  INT4 weights are
// unpacked to INT8 before the INT8 matmul ("cider" post, modes table).
//
// Design (CDNA4, wave64; the per-channel large tiles run one wave per SIMD,
// the per-group ones two):
//  * One workgroup computes BM x BN tiles of Y (m x n) with WM x WN waves.
//    Both operands are K-contiguous.  v_mfma_i32_32x32x32_i8 multiplies two
//    32 x 32-k fragments (16 bytes per lane each); a lane of its result holds
//    one column of the first operand's transpose and runs of four rows.  The
//    per-channel path puts the weights first, so a lane holds one output row
//    m and runs of four consecutive columns n, which become 8-byte fp16 runs
//    (16 bytes after one cross-half lane swap) with no other shuffling; the
//    per-group and int32 paths put the activations first (one column n, runs
//    of rows m), which matches their per-column scales and int32 stores.
//    This MFMA sustains close to the int8 peak with a single wave per SIMD,
//    which the large per-wave tiles need (they keep LDS reads per MFMA low).
//  * K advances in stages of 128 bytes through a ring of R = 3 LDS buffers
//    (R = 4 for the few-token per-channel tiles).
//    Stages are copied from global memory straight into LDS (buffer loads
//    with the lds modifier, 16-byte chunks XOR-swizzled per row); the copies
//    of one stage are spread over four k-steps between the MFMAs, and the
//    only waits are explicit vmcnt counts before an LDS-only barrier.
//  * Per-tile buffer resources make rows past the end of X or W read as
//    zeros, so copies need no per-lane clamping.
//  * The kernel is persistent: each workgroup walks a list of tiles and its
//    stages form one stream across them, so the next tile's first stages are
//    in flight while the current one finishes.
//  * int4 weights are loaded packed (half the bytes), unpacked in registers to
//    16 * code (the nibble placed in the high half of each byte, which is
//    the code times 16 as a signed byte) and stored to LDS in the same int8
//    layout; the factor 16 is undone in the epilogue (exact).
//  * Per-group modes restart the int32 accumulators for every group and fold
//    them into fp32 accumulators with the group's scales, which are staged
//    through LDS together with the tiles (in a ring of their own).  Their
//    large tiles run two waves per SIMD: the fold is VALU work that does not
//    overlap the MFMAs of its own wave, only those of the other wave.
//  * Workgroups are renumbered so that each XCD (one L2 each) works on a
//    contiguous range of tiles, ordered in groups of `group_m` tile rows.
#include <type_traits>

#include "kernels.hpp"
#include "lds_copy.hpp"

namespace w4a8 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 128;          // k bytes per LDS stage (four 32-wide MFMA steps)

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row r (rows are
// 128 bytes).  A 16-byte-per-lane LDS read serves 16 lanes per cycle from 64
// four-byte banks, i.e. two rows' worth; fragment reads put 16 consecutive
// rows, one logical chunk each, in such a group.  XOR with r & 7 spreads
// 8 rows over the 8 chunk positions, and the extra flip for rows 8..15 moves
// them to the other half of the banks' 16-byte slots, so all 16 lanes hit
// distinct banks (and any 8 consecutive lanes still do).  An involution in
// c for fixed r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Unpack 8 int4 codes (one dword, low nibble = even k) into 8 signed bytes
// holding 16 * code, in natural k order (two dwords).
__device__ __forceinline__ uint2 unpack_int4x8(uint32_t x)
{
    const uint32_t lo = (x << 4) & 0xf0f0f0f0u;   // k = 0, 2, 4, 6  (times 16)
    const uint32_t hi = x & 0xf0f0f0f0u;          // k = 1, 3, 5, 7  (times 16)
    // interleave bytes: {lo0, hi0, lo1, hi1} and {lo2, hi2, lo3, hi3}
    const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    return make_uint2(a, b);
}

// Output pairs.  Each lane holds, for one output column n, the values of two
// consecutive rows m, m+1 (packed as fp16 lo/hi).  Adjacent lanes (n even,
// n+1) trade halves so that the even lane holds row m at columns n, n+1 and
// the odd lane row m+1 at columns n-1, n: one 4-byte store each.
__device__ __forceinline__ uint32_t pair_rows_to_cols(uint32_t p, uint32_t sel)
{
    // the neighbouring lane's pair (quad_perm [1, 0, 3, 2])
    const uint32_t q = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0xb1, 0xf, 0xf, false);
    return __builtin_amdgcn_perm(p, q, sel);
}

template <GemmMode MODE> struct ModeTraits {
    static constexpr bool int4 = (MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool pergroup = (MODE == GemmMode::PG || MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool partials = (MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4_PARTIALS);
    static constexpr bool fold_sa = (MODE == GemmMode::PG);     // per-group activation scales
    static constexpr bool fold_sw = (MODE == GemmMode::PG || MODE == GemmMode::W4);
    // weights as the MFMA's first operand: lane = output row, runs along n
    static constexpr bool nmajor = (MODE == GemmMode::PC);
};

// Persistent kernel: the grid holds at most as many workgroups as fit on the
// device at once, and workgroup b computes the tiles b', b' + G, b' + 2G, ...
// of a fixed tile order (G = grid size, b' an XCD-contiguous renumbering of
// b).  Its K-stages form one stream across its tiles, so the copies of the
// next tile's first stages are in flight while the current tile finishes and
// writes its outputs.
// Size of the p-th non-empty window of w[0..3] (0 past the last one).
constexpr int part_of_windows(const int (&w)[4], int p)
{
    for (int i = 0; i < 4; ++i)
        if (w[i] != 0 && p-- == 0)
            return w[i];
    return 0;
}

template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(GemmArgs args, int tiles_m,
                                                           int tiles_n, int group_m)
{
    using T = ModeTraits<MODE>;
    constexpr int NW = WM * WN;                       // waves
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    constexpr int XBUF = BM * BK, WBUF = BN * BK;
    // direct-to-LDS copies: one wave instruction moves 1 KiB = 8 rows of a stage
    constexpr int XB = XBUF / 1024 / NW;              // X blocks per wave per stage
    static_assert(XBUF % (1024 * NW) == 0, "X stage must split evenly over the waves");
    constexpr bool kDmaW = !T::int4;                  // int8 weights go straight to LDS
    constexpr int WB = kDmaW ? WBUF / 1024 / NW : 0;
    static_assert(!kDmaW || WBUF % (1024 * NW) == 0, "W stage must split evenly over the waves");
    // packed int4 weights are staged through registers and unpacked
    constexpr int WCH4 = BN * 4;                      // 16-byte packed chunks per stage
    constexpr int WIT4 = T::int4 ? (WCH4 + NW * 64 - 1) / (NW * 64) : 0;
    constexpr int NG = T::pergroup ? BK / GS : 1;     // groups per stage
    constexpr int SPG = T::pergroup ? GS / 32 : 4;    // k-steps per group
    // scale copies (4 bytes per lane): per stage NG*BM activation scales and
    // NG*BN weight scales, in instructions of 64 lanes, dealt round-robin
    constexpr int SA_I = T::fold_sa ? (NG * BM + 63) / 64 : 0;
    constexpr int SW_I = T::fold_sw ? (NG * BN + 63) / 64 : 0;
    constexpr int SAW = (SA_I + NW - 1) / NW, SWW = (SW_I + NW - 1) / NW;
    // copy instructions of one stage, per wave: X blocks, W blocks, then the
    // scale instructions (which some waves skip where they do not split evenly)
    constexpr int NCW = XB + WB + SAW + SWW;
    // copies every wave surely issues per stage (waiting on it is exact or
    // conservative)
    constexpr int ND = XB + WB + SA_I / NW + SW_I / NW;
    // The copies of stage u are spread over four k-steps: part A in step 3 of
    // iteration u-R, parts 0..2 in steps 0..2 of iteration u-R+1 (R, the LDS
    // ring depth, is 3 except for the few-token tiles below).  Scale copies
    // never go in part A (the group fold after step 3 still reads the scales
    // in that buffer).  int4 weights are register-staged; their compiler
    // tracked loads make it wait for every earlier copy before the unpack, so
    // there the tile copies all go in part A and the scale copies in part 0.
    // Tile copies go in windows of up to four consecutive 1 KiB blocks that
    // share one M0 value (see issue_copy); without scale copies each part is
    // one window: X blocks 0-3, X 4-7, W 0-3, W 4-7 (empty windows dropped).
    constexpr int NCP = NCW / 4, NCR = NCW % 4;
    constexpr bool WSPLIT = !T::pergroup && !T::int4 && XB <= 8 && WB <= 8;
    constexpr int WIN[4] = {XB < 4 ? XB : 4, XB < 4 ? 0 : XB - 4, WB < 4 ? WB : 4, WB < 4 ? 0 : WB - 4};
    constexpr int CA = WSPLIT ? part_of_windows(WIN, 0) : T::int4 ? XB + WB : NCP + (NCR > 0);
    constexpr int C0 = WSPLIT ? part_of_windows(WIN, 1) : T::int4 ? NCW - CA : NCP + (NCR > 1);
    constexpr int C1 = WSPLIT ? part_of_windows(WIN, 2) : T::int4 ? 0 : NCP + (NCR > 2);
    constexpr int C2 = WSPLIT ? part_of_windows(WIN, 3) : T::int4 ? 0 : NCP;
    static_assert(CA + C0 + C1 + C2 == NCW, "copy split");
    static_assert(!T::pergroup || CA <= XB + WB, "scale copies must not go in part A");
    // epilogue scales staged in LDS: per-token sa (PC, W4) followed by
    // per-channel sw (PC)
    constexpr int ESN = (MODE == GemmMode::PC) ? BM + BN : (MODE == GemmMode::W4 ? BM : 0);
    constexpr int EW = (ESN + 64 * NW - 1) / (64 * NW);   // copy instructions per wave

    // LDS ring depth: three stages, four for the few-token per-channel tiles
    // (their stages are small, and one more stage in flight shortens the
    // waits on weights that come from HBM)
    constexpr int RING = (!T::pergroup && !T::int4 && BN <= 64) ? 4 : 3;
    static_assert((RING - 2) * ND + CA < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) int8_t xs[RING * XBUF];
    __shared__ __attribute__((aligned(1024))) int8_t ws[RING * WBUF];
    // Group scales have a ring of their own, one slot per stage: a group is
    // folded after its last k-step, which for the last group of a stage comes
    // after the barrier of its iteration, while a wave that is already past
    // that barrier issues the scale copies of stages up to three ahead.
    constexpr int SR = 5;                             // scale ring slots
    constexpr int SAL = T::fold_sa ? NG * BM : 1, SWL = T::fold_sw ? NG * BN : 1;
    __shared__ __attribute__((aligned(16))) float sas[T::fold_sa ? SR * SAL : 1];
    __shared__ __attribute__((aligned(16))) float sws[T::fold_sw ? SR * SWL : 1];
    __shared__ __attribute__((aligned(16))) float eps[EW > 0 ? EW * NW * 64 : 1];

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- this workgroup's tiles.  Workgroups are dealt to the XCDs round
    // robin; renumber them so each XCD holds a contiguous range, and order the
    // tiles in groups of group_m tile rows, so that the tiles in flight on one
    // XCD (one L2) share rows of X and of W.
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
        m0 = (first_m + in % gm) * BM;
        n0 = (in / gm) * BN;
    };
    const int G_ = T::pergroup ? K / GS : 1;          // groups along K
    const int nstage = (K + BK - 1) / BK;
    const int nks = K / 32;                           // 32-wide MFMA steps in K
    const int U = ntile * nstage;                     // stages this workgroup computes

    const int8_t *__restrict__ xq = args.xq;
    const uint8_t *__restrict__ wb = static_cast<const uint8_t *>(args.w);
    const int wrow = T::int4 ? K / 2 : K;             // bytes per weight row

    // Direct-to-LDS copies.  A wave instruction writes lane l's 16 bytes at
    // LDS block + 16*l, i.e. row 8*blk + l/8, physical chunk l%8; the lane
    // therefore fetches the logical chunk that the swizzle puts there.  Wave w
    // copies the X blocks w*XB .. w*XB + XB - 1 of a stage and the W blocks
    // w*WB .., in windows of four blocks (32 rows) whose copies share one M0
    // value: copy q of a window reaches its block through the instruction
    // offset 1024 q, which moves the global address by the same amount, so
    // the lane offset carries -1024 q (whole stages; with a K tail the
    // offset is 0 and M0 moves per copy).  Window h adds 32 h rows to the
    // lane offset.  Byte offsets within a tile; rows past the end of the
    // matrix fall outside the tile's buffer resource (the instruction offset
    // takes part in the range check) and read as zeros.
    const int dma_row = lane >> 3;
    auto lane_off = [&](int nb, int q, bool shifted) __attribute__((always_inline)) {
        // row 8 (w*nb + q) + l/8 of the tile, the swizzle parity of block w*nb + q
        const int row = (wave * nb + q) * 8 + dma_row;
        const int c = (lane & 7) ^ dma_row ^ ((wave * nb + q) & 1);
        return (uint32_t)(row * K + c * 16 - (shifted ? 1024 * q : 0));
    };
    uint32_t vqx[XB < 4 ? XB : 4], vqw[WB == 0 ? 1 : (WB < 4 ? WB : 4)];
    const bool kwhole = K % BK == 0;
#pragma unroll
    for (int q = 0; q < (XB < 4 ? XB : 4); ++q)
        vqx[q] = lane_off(XB, q, kwhole);
#pragma unroll
    for (int q = 0; q < (WB < 4 ? WB : 4); ++q)
        vqw[q] = lane_off(WB, q, kwhole);

    // Where the copies of one stage come from: the stage's tile, its index
    // within the tile and the LDS buffer it goes to.  Wave-uniform.
    struct Src {
        int v;         // stage in this workgroup's stream (clamped to U - 1)
        int s;         // stage within its tile
        int tile;      // tile within this workgroup's list
        int buf;       // LDS buffer (the unclamped stage index mod RING)
        int sb;        // scale ring slot (the unclamped stage index mod SR)
        int m0, n0;    // tile origin
        v4i rx, rw;    // buffer resources of the tile's X rows and int8 W rows
    };
    auto set_tile = [&](Src &c, int i) __attribute__((always_inline)) {
        c.tile = i;
        tile_origin(i, c.m0, c.n0);
        c.rx = make_rsrc(xq + (int64_t)c.m0 * K, (uint32_t)(min(BM, M - c.m0) * K));
        if constexpr (kDmaW)
            c.rw = make_rsrc(wb + (int64_t)c.n0 * K, (uint32_t)(min(BN, N - c.n0) * K));
    };
    auto advance = [&](Src &c) __attribute__((always_inline)) {
        c.buf = c.buf == RING - 1 ? 0 : c.buf + 1;
        c.sb = c.sb == SR - 1 ? 0 : c.sb + 1;
        if (c.v + 1 < U) {                            // past the end: repeat the last stage
            ++c.v;
            if (++c.s == nstage) {
                c.s = 0;
                set_tile(c, c.tile + 1);
            }
        }
    };

    // Copy c (0 <= c < NCW) of the stage described by `src`.  c is a
    // constant once the callers' loops are unrolled.
    // The stage's K offset goes in the scalar offset when K % 128 == 0 (every
    // stage is whole, so a row's bytes never run past its end); for a K tail
    // it is added to the per-lane offset, which the resource's range check
    // covers.  `first`: the first copy of a run (M0 is set again).
    auto issue_copy = [&](const Src &src, int buf, int c, bool first, auto KFULL)
                          __attribute__((always_inline)) {
        constexpr bool kfull = decltype(KFULL)::value;
        const uint32_t k0 = (uint32_t)(src.s * BK);
        if (c < XB + WB) {
            const bool isx = c < XB;
            const int nb = isx ? XB : WB;
            const int i = isx ? c : c - XB;
            const int q = i % 4, h = i / 4;
            const int blk0 = wave * nb + 4 * h;       // the window's first block
            const v4i r = isx ? src.rx : src.rw;
            const uint32_t lds = lds_addr((isx ? xs + buf * XBUF : ws + buf * WBUF) + blk0 * 1024);
            const uint32_t voff = (isx ? vqx[q] : vqw[q]) + (uint32_t)(h * 32 * K);
            if constexpr (kfull) {
                if (first || q == 0)
                    set_m0(lds);
                if (q == 0)
                    copy16_buf_to_lds<0>(r, voff, k0);
                else if (q == 1)
                    copy16_buf_to_lds<1024>(r, voff, k0);
                else if (q == 2)
                    copy16_buf_to_lds<2048>(r, voff, k0);
                else
                    copy16_buf_to_lds<3072>(r, voff, k0);
            } else {
                set_m0(lds + 1024 * q);
                copy16_buf_to_lds<0>(r, voff + k0, 0u);
            }
        } else if (c < XB + WB + SAW) {
            if constexpr (T::fold_sa) {
                const int ins = wave + NW * (c - XB - WB);
                if (SA_I % NW == 0 || ins < SA_I) {
                    const int e = ins * 64 + lane;    // entry g*BM + r
                    const int g = min(e / BM, NG - 1), r = e % BM;
                    const int gi = min(src.s * NG + g, G_ - 1);
                    if (e < NG * BM)
                        copy4_to_lds(args.sa + (int64_t)min(src.m0 + r, M - 1) * G_ + gi,
                                     lds_addr(sas + src.sb * SAL + ins * 64));
                }
            }
        } else {
            if constexpr (T::fold_sw) {
                const int ins = wave + NW * (c - XB - WB - SAW);
                if (SW_I % NW == 0 || ins < SW_I) {
                    const int e = ins * 64 + lane;    // entry g*BN + r
                    const int g = min(e / BN, NG - 1), r = e % BN;
                    const int gi = min(src.s * NG + g, G_ - 1);
                    if (e < NG * BN)
                        copy4_to_lds(args.sw + (int64_t)min(src.n0 + r, N - 1) * G_ + gi,
                                     lds_addr(sws + src.sb * SWL + ins * 64));
                }
            }
        }
    };
    // Copies [c0, c0 + n) of a stage, back to back.
    auto issue_copies = [&](const Src &src, int buf, int c0, int n, auto KFULL)
                            __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCW; ++c)
            if (c >= c0 && c < c0 + n)
                issue_copy(src, buf, c, c == c0, KFULL);
    };
    // The epilogue scales of the tile at (m0, n0); rows and columns past the
    // end repeat the last one.
    auto issue_epilogue_scales = [&](int m0, int n0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < EW; ++i) {
            const int e = (wave + NW * i) * 64 + lane;
            const float *src;
            if (e < BM)
                src = args.sa + min(m0 + e, M - 1);
            else if (MODE == GemmMode::PC && e < BM + BN)
                src = args.sw + min(n0 + e - BM, N - 1);
            else
                src = args.sa + min(m0, M - 1);        // padding slot, never read
            copy4_to_lds(src, lds_addr(eps + (wave + NW * i) * 64));
        }
    };

    // ---- packed int4 weights: register staging and unpack into LDS
    uint4 w4r[WIT4 > 0 ? WIT4 : 1];
    auto w4_load = [&](const Src &src) __attribute__((always_inline)) {
        const int kb0 = src.s * (BK / 2);
#pragma unroll
        for (int it = 0; it < WIT4; ++it) {
            const int q = min(tid + it * NW * 64, WCH4 - 1);
            const int c = q & 3;
            const bool ok = kb0 + c * 16 < wrow;
            const int64_t off = (int64_t)min(src.n0 + (q >> 2), N - 1) * wrow + c * 16;
            w4r[it] = *reinterpret_cast<const uint4 *>(wb + off + (ok ? kb0 : wrow - 16 - c * 16));
        }
    };
    auto w4_store = [&](int buf) __attribute__((always_inline)) {
        int8_t *W = ws + buf * WBUF;
#pragma unroll
        for (int it = 0; it < WIT4; ++it) {
            const int q = tid + it * NW * 64;
            if (WCH4 % (NW * 64) == 0 || q < WCH4) {
                const int row = q >> 2, c = q & 3;    // packed chunk c -> int8 chunks 2c, 2c+1
                const uint2 a = unpack_int4x8(w4r[it].x), b = unpack_int4x8(w4r[it].y);
                const uint2 d = unpack_int4x8(w4r[it].z), e = unpack_int4x8(w4r[it].w);
                *reinterpret_cast<uint4 *>(W + row * BK + swz(row, 2 * c) * 16) =
                    make_uint4(a.x, a.y, b.x, b.y);
                *reinterpret_cast<uint4 *>(W + row * BK + swz(row, 2 * c + 1) * 16) =
                    make_uint4(d.x, d.y, e.x, e.y);
            }
        }
    };

    // ---- accumulators: acc[j][i] is the 32x32 block (n-block j, m-block i)
    v16i acc[FN][FM];
    v16f accf[T::fold_sw ? FN : 1][T::fold_sw ? FM : 1];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
            acc[j][i] = v16i{};
    auto clear_accf = [&]() __attribute__((always_inline)) {
        if constexpr (T::fold_sw) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    accf[j][i] = v16f{};
        }
    };
    clear_accf();

    // Fragment addressing: lane reads row (base + lane%32), logical chunk
    // 2t + lane/32 for k-step t; bases are multiples of 32, so the swizzle
    // depends on lane%32 only.
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;
    int fo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        fo[t] = lrow * BK + swz(lrow, 2 * t + lhalf) * 16;
    const int xrow0 = wm * TM;
    const int wrow0 = wn * TN;
    // output coordinates of this lane inside a 32x32 block: n = lane%32,
    // m = 8*(r/4) + 4*(lane/32) + r%4 for accumulator element r
    const int out_n = lane & 31;
    const int out_m = lhalf * 4;
    // byte selector of pair_rows_to_cols: even lanes keep the low halves
    // (row m), odd lanes the high halves (row m+1)
    const uint32_t pair_sel = (lane & 1) ? 0x07060302u : 0x01000504u;

    struct Frag {
        v4i a[FN];    // weights (B operand)
        v4i b[FM];    // activations (A operand)
    };
    Frag f0, f1;

    // Fragment r (0 <= r < FM + FN) of k-step t from buffer buf, in the order
    // the next step's MFMAs first use them: b[0], a[0], b[1..], a[1..].
    constexpr int NR = FM + FN;
    auto read_one = [&](Frag &F, int buf, int t, int r) __attribute__((always_inline)) {
        const int8_t *xb = xs + buf * XBUF + xrow0 * BK + fo[t];
        const int8_t *wbf = ws + buf * WBUF + wrow0 * BK + fo[t];
        if (r == 0)
            F.b[0] = *reinterpret_cast<const v4i *>(xb);
        else if (r == 1)
            F.a[0] = *reinterpret_cast<const v4i *>(wbf);
        else if (r < FM + 1)
            F.b[r - 1] = *reinterpret_cast<const v4i *>(xb + (r - 1) * 32 * BK);
        else
            F.a[r - FM] = *reinterpret_cast<const v4i *>(wbf + (r - FM) * 32 * BK);
    };
    auto read_frag = [&](Frag &F, int buf, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
            read_one(F, buf, t, r);
    };

    // Fold (per-group modes): the group's int32 sums, rescaled by the group's
    // scales, are added to the fp32 accumulators.  Chunk c = (m-block i, row
    // quad q) covers elements 4q..4q+3 of blocks (j, i) for every j and
    // needs the four activation scales of those rows.  The group's scales
    // are read from its stage's slot of the scale ring.
    constexpr int NCH = FM * 4;
    auto fold_group = [&](int slot, int g) __attribute__((always_inline)) {
        float fsw[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fsw[j] = sws[slot * SWL + g * BN + wn * TN + j * 32 + out_n];
        v4f fsa = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int i = c / 4, q = c % 4;
            if constexpr (T::fold_sa)
                fsa = *reinterpret_cast<const v4f *>(&sas[slot * SAL + g * BM + wm * TM + i * 32 + q * 8 + out_m]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sc = T::fold_sa ? fsa[r] * fsw[j] : fsw[j];
                    accf[j][i][4 * q + r] = fmaf((float)acc[j][i][4 * q + r], sc, accf[j][i][4 * q + r]);
                }
        }
    };

    // The MFMAs of one k-step (restarting the sums when RESTART) on F.
    // Interleaved with them: the fragments of the next step into G (fragment
    // r after MFMA r * FN * FM / (2 NR): all within the first half of the
    // step, so they have landed when the next step starts), and copies
    // [c0, c0 + n) of the stage `src` (copy p after MFMA (2p + 1) * FN * FM / (2n)).
    auto mfma_step = [&](const Frag &F, auto RESTART, Frag &G, bool reads, int rbuf, int rt,
                         const Src &src, int sbuf, int c0, int n, auto KFULL)
                         __attribute__((always_inline)) {
        constexpr bool restart = decltype(RESTART)::value;
        constexpr int NM = FN * FM;
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const int j = k / FM, i = k % FM;
            if constexpr (T::nmajor)
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.a[j], F.b[i],
                                                                  restart ? v16i{} : acc[j][i], 0, 0, 0);
            else
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.b[i], F.a[j],
                                                                  restart ? v16i{} : acc[j][i], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (reads) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if ((r * NM) / (2 * NR) == k)
                        read_one(G, rbuf, rt, r);
            }
#pragma unroll
            for (int p = 0; p < NCW; ++p)
                if (p < n && k == ((2 * p + 1) * NM) / (2 * n))
                    issue_copy(src, sbuf, c0 + p, p == 0, KFULL);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // int32 sums of a 32x32 block: per accumulator element one 4-byte store,
    // lanes 0-31 along one row, 32-63 along the row four below.
    auto store_block_i32 = [&](int32_t *C, const v16i &blk, int mb, int nb, bool shift4)
                               __attribute__((always_inline)) {
        const int n = nb + out_n;
        if (n >= N)
            return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = mb + 8 * (r / 4) + out_m + r % 4;
            if (m < M)
                C[(int64_t)m * N + n] = shift4 ? (blk[r] >> 4) : blk[r];
        }
    };
    auto store_partials = [&](int m0, int n0, int g) __attribute__((always_inline)) {
        int32_t *P = static_cast<int32_t *>(args.out) + (int64_t)g * M * N;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)   // int4: exact, the sums are 16 * P
                store_block_i32(P, acc[j][i], m0 + wm * TM + i * 32, n0 + wn * TN + j * 32, T::int4);
    };

    // ---- the tile's outputs from the final sums
    auto epilogue = [&](int m0, int n0) __attribute__((always_inline)) {
        if constexpr (MODE == GemmMode::I32) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    store_block_i32(static_cast<int32_t *>(args.out), acc[j][i],
                                    m0 + wm * TM + i * 32, n0 + wn * TN + j * 32, false);
        } else if constexpr (T::nmajor) {
            // Lane l holds row m = mw + 32 i + l % 32 of block (i, j); its
            // accumulator elements 4g..4g+3 are columns nb + 8g + 4 (l / 32) + 0..3.
            uint16_t *Y = static_cast<uint16_t *>(args.out);
            const int mw = m0 + wm * TM, nw = n0 + wn * TN;
            const int lr = lane & 31, lh = lane >> 5;
            float sam[FM];                       // sa of this lane's rows (clamped at M - 1)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                sam[i] = eps[wm * TM + i * 32 + lr];
            // whole tile inside the output, rows a multiple of 16 bytes long
            // and a 16-byte aligned output: every 16-byte store is in bounds
            // and aligned
            const bool fast = m0 + BM <= M && n0 + BN <= N && (N & 7) == 0 &&
                              ((uintptr_t)Y & 15) == 0;
            if (fast) {
                // lane's 16-byte piece of a 16-column half row: row lr,
                // columns 8 lh .. 8 lh + 7 of the half
                const uint32_t voff = (uint32_t)((lr * N + 8 * lh) * 2);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    v4f swv[4];                  // sw of columns nb + 8g + 4 lh + 0..3
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        swv[g] = *reinterpret_cast<const v4f *>(
                            &eps[BM + wn * TN + j * 32 + 8 * g + 4 * lh]);
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        uint32_t d[8];           // fp16 pairs, columns 8g + 4 lh + {0,1}, {2,3}
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            float v[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                v[r] = rescale_pc(acc[j][i][4 * g + r], sam[i], swv[g][r]);
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
                        // wave-uniform block base plus the lane's 32-bit offset
                        char *blk = reinterpret_cast<char *>(
                            Y + (int64_t)(mw + i * 32) * N + nw + j * 32) + voff;
                        *reinterpret_cast<v4u *>(blk) = v4u{d[0], d[1], d[2], d[3]};
                        *reinterpret_cast<v4u *>(blk + 32) = v4u{d[4], d[5], d[6], d[7]};
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int m = mw + i * 32 + lr;
                        if (m < M) {
#pragma unroll
                            for (int g = 0; g < 4; ++g)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int nl = wn * TN + j * 32 + 8 * g + 4 * lh + r;
                                    if (n0 + nl < N)
                                        Y[(int64_t)m * N + n0 + nl] =
                                            f2h(rescale_pc(acc[j][i][4 * g + r], sam[i], eps[BM + nl]));
                                }
                        }
                    }
            }
        } else if constexpr (!T::partials) {
            uint16_t *Y = static_cast<uint16_t *>(args.out);
            // whole tile inside the output and rows of an even length: every
            // pair store is in bounds and 4-byte aligned
            const bool fast = m0 + BM <= M && n0 + BN <= N && (N & 1) == 0;
            // this lane's store position relative to a pair of rows: even
            // lanes write row m at columns n, n+1; odd lanes row m+1 at n-1, n
            const uint32_t lane_off =
                (uint32_t)(((out_m + (lane & 1)) * N + out_n - (lane & 1)) * 2);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mb = m0 + wm * TM + i * 32;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // per-token scales of rows mb + 8q + out_m + 0..3
                    v4f sav = {1.0f, 1.0f, 1.0f, 1.0f};
                    if constexpr (MODE != GemmMode::PG)
                        sav = *reinterpret_cast<const v4f *>(&eps[wm * TM + i * 32 + q * 8 + out_m]);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int nb = n0 + wn * TN + j * 32;
                        float v[4];
                        if constexpr (MODE == GemmMode::PG) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                v[r] = accf[j][i][4 * q + r];
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)   // W4: per-token scale, undo x16 (exact)
                                v[r] = accf[j][i][4 * q + r] * (sav[r] * 0.0625f);
                        }
                        if (fast) {
#pragma unroll
                            for (int h = 0; h < 2; ++h) {    // rows mb + 8q + out_m + 2h (+1)
                                const uint32_t w = pair_rows_to_cols(pack_h2(v[2 * h], v[2 * h + 1]),
                                                                     pair_sel);
                                // wave-uniform row base plus the lane's 32-bit offset
                                char *row = reinterpret_cast<char *>(
                                    Y + (int64_t)(mb + q * 8 + 2 * h) * N + nb);
                                *reinterpret_cast<uint32_t *>(row + lane_off) = w;
                            }
                        } else {
                            const int m = mb + q * 8 + out_m, n = nb + out_n;
                            if (n < N) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (m + r < M)
                                        Y[(int64_t)(m + r) * N + n] = f2h(v[r]);
                            }
                        }
                    }
                    // a quarter of the sums at a time: keeps the reads of
                    // the others from being hoisted here
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // ---- pipeline.  Stage u of the stream lives in LDS buffer u % R (R =
    // RING).  Its copies are issued in four parts: part A during step 3 of
    // iteration u-R, right after the barrier that frees the buffer, and parts
    // 0-2 during steps 0-2 of iteration u-R+1 (int4 weights, R = 3: loaded
    // into registers in iteration u-2 and unpacked to LDS before the barrier
    // of iteration u-1).  Iteration u: steps 0-2 from buffer u%R; wait for
    // stage u+1 (the R-2 later stages' copies may stay in flight) and
    // barrier; step 3, which also reads the first fragments of stage u+1;
    // after the last stage of a tile, its epilogue.  Every iteration issues
    // the same copies -- past the end of the stream they repeat the last
    // stage into a buffer nobody reads -- so every wait count is a constant.
    auto main_loop = [&](auto KFULL) __attribute__((always_inline)) {
        constexpr bool kfull = decltype(KFULL)::value;   // K % 128 == 0: every k-step exists
        Src cp;                                       // stages 0 .. R-1 (prologue)
        cp.v = 0; cp.s = 0; cp.buf = 0; cp.sb = 0;
        set_tile(cp, 0);
        int cm0 = cp.m0, cn0 = cp.n0, ctile = 0;      // the tile being computed
        if constexpr (EW > 0)
            issue_epilogue_scales(cm0, cn0);          // complete before stage 0 does
        issue_copies(cp, cp.buf, 0, NCW, KFULL);
        if constexpr (T::int4) {
            w4_load(cp);
            w4_store(0);
        }
        advance(cp);
        if constexpr (T::int4)
            w4_load(cp);
        issue_copies(cp, cp.buf, 0, NCW, KFULL);
        advance(cp);
#pragma unroll
        for (int e = 3; e < RING; ++e) {              // stages 2 .. RING - 2
            issue_copies(cp, cp.buf, 0, NCW, KFULL);
            advance(cp);
        }
        issue_copies(cp, cp.buf, 0, CA, KFULL);
        Src c2 = cp;                                  // stage u+R-1: parts 0-2 in iteration u
        advance(cp);
        Src c3 = cp;                                  // stage u+R: part A in iteration u
        wait_vmcnt<(RING - 2) * ND + CA>();
        lds_barrier();
        read_frag(f0, 0, 0);

        int b = 0, s = 0;                             // buffer and in-tile stage of iteration u
        int sb = 0;                                   // scale ring slot of iteration u
        for (int u = 0; u < U; ++u) {
            const int b1 = b == RING - 1 ? 0 : b + 1;
            const int ks0 = s * 4;
            auto step = [&](auto TC, const Src &src, int c0, int n) __attribute__((always_inline)) {
                constexpr int t = decltype(TC)::value;
                Frag &cur = (t & 1) ? f1 : f0;
                Frag &nxt = (t & 1) ? f0 : f1;
                if (kfull || ks0 + t < nks) {
                    // the next step's fragments: of this stage, or (step 3)
                    // of the next stage (which nothing overwrites before it
                    // is computed, also across a tile's epilogue)
                    const bool reads = t < 3 ? (kfull || ks0 + t + 1 < nks) : true;
                    const int rbuf = t < 3 ? b : b1, rt = (t + 1) & 3;
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (T::pergroup) {
                        if constexpr (t % SPG == 0)
                            mfma_step(cur, std::true_type(), nxt, reads, rbuf, rt, src, src.buf, c0,
                                      n, KFULL);
                        else
                            mfma_step(cur, std::false_type(), nxt, reads, rbuf, rt, src, src.buf, c0,
                                      n, KFULL);
                    } else if constexpr (t == 0) {
                        if (s == 0)                   // a tile's first k-step
                            mfma_step(cur, std::true_type(), nxt, reads, rbuf, rt, src, src.buf, c0,
                                      n, KFULL);
                        else
                            mfma_step(cur, std::false_type(), nxt, reads, rbuf, rt, src, src.buf, c0,
                                      n, KFULL);
                    } else {
                        mfma_step(cur, std::false_type(), nxt, reads, rbuf, rt, src, src.buf, c0, n,
                                  KFULL);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // close a group where one ends (groups are whole runs of
                    // k-steps: K % gs == 0)
                    if constexpr (T::pergroup && (t + 1) % SPG == 0) {
                        if constexpr (T::partials)
                            store_partials(cm0, cn0, s * NG + t / SPG);
                        else
                            fold_group(sb, t / SPG);
                    }
                } else {
                    // a K % 128 == 64 tail: the step does not exist, its copies
                    // (and after the barrier the next stage's fragments) do
                    if constexpr (t == 3)
                        read_frag(nxt, b1, 0);
                    issue_copies(src, src.buf, c0, n, KFULL);
                }
            };
            step(std::integral_constant<int, 0>(), c2, CA, C0);
            step(std::integral_constant<int, 1>(), c2, CA + C0, C1);
            step(std::integral_constant<int, 2>(), c2, CA + C0 + C1, C2);
            // stage u+1 complete and visible; buffer b free
            if constexpr (T::int4)
                w4_store(b1);
            wait_vmcnt<(RING - 2) * ND>();
            lds_barrier();
            if constexpr (T::int4)
                w4_load(c2);
            step(std::integral_constant<int, 3>(), c3, 0, CA);

            if (s + 1 == nstage) {                    // the tile is done
                if constexpr (EW > 0) {
                    if (nstage < RING) {              // its scales may still be in flight
                        wait_vmcnt<0>();
                        lds_barrier();
                    }
                }
                epilogue(cm0, cn0);
                clear_accf();
                s = 0;
                if (++ctile < ntile) {
                    tile_origin(ctile, cm0, cn0);
                    if constexpr (EW > 0) {
                        lds_barrier();                // every wave is done with the scales
                        issue_epilogue_scales(cm0, cn0);
                    }
                }
            } else {
                ++s;
            }
            c2 = c3;
            advance(c3);
            b = b1;
            sb = sb == SR - 1 ? 0 : sb + 1;
        }
        // no copy may still be writing LDS when the workgroup ends
        wait_vmcnt<0>();
    };
    if (K % BK == 0)
        main_loop(std::true_type());
    else
        main_loop(std::false_type());
}

// Workgroups of one instantiation that fit on a compute unit at once.
template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS>
int groups_per_cu()
{
    static const int occ = [] {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_kernel<BM, BN, WM, WN, MODE, GS>,
                                                         WM * WN * 64, 0) != hipSuccess || o < 1)
            o = 1;
        return o;
    }();
    return occ;
}

template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS>
void launch_cfg(const GemmArgs &a, hipStream_t st)
{
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int group_m = 4;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t resident = (int64_t)a.num_cu * groups_per_cu<BM, BN, WM, WN, MODE, GS>();
    const unsigned grid = (unsigned)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, GS>), dim3(grid), dim3(WM * WN * 64), 0, st,
                       a, tiles_m, tiles_n, group_m);
}

// Tile shapes choose_tile can return for a mode (only these are compiled).
template <GemmMode MODE, int GS> constexpr bool tile_ok(TileShape t)
{
    using T = ModeTraits<MODE>;
    constexpr bool pg64 = (MODE == GemmMode::PG || MODE == GemmMode::PG_PARTIALS) && GS == 64;
    switch (t) {
    case TileShape::T32x32: return !T::int4;
    case TileShape::T32x128: return T::int4;
    case TileShape::T64x64: return !T::pergroup;
    case TileShape::T64x128: return true;
    case TileShape::T128x128: return true;
    case TileShape::T128x128w8: return pg64;
    case TileShape::T256x128: return !T::pergroup;
    case TileShape::T256x128w8: return T::pergroup && !pg64;
    case TileShape::T256x160: return !T::pergroup;
    case TileShape::T128x160: return !T::pergroup;
    case TileShape::T256x320w8: return false;       // a kernel of its own
    case TileShape::TSkinny: return false;          // a kernel of its own
    case TileShape::TRows: return false;            // a kernel of its own
    }
    return false;
}

// F<BM, BN, WM, WN, MODE, GS>::run(args...) for the runtime tile t.
template <GemmMode MODE, int GS, template <int, int, int, int, GemmMode, int> class F, typename... A>
int with_tile(TileShape t, A &&...args)
{
#define W4A8_TILE(S, BM, BN, WM, WN)                                                 \
    case TileShape::S:                                                              \
        if constexpr (tile_ok<MODE, GS>(TileShape::S))                              \
            return F<BM, BN, WM, WN, MODE, GS>::run(args...);                       \
        return -1;
    switch (t) {
        W4A8_TILE(T32x32, 32, 32, 1, 1)
        W4A8_TILE(T32x128, 32, 128, 1, 4)
        W4A8_TILE(T64x64, 64, 64, 1, 2)
        W4A8_TILE(T64x128, 64, 128, 2, 2)
        W4A8_TILE(T128x128, 128, 128, 2, 2)
        W4A8_TILE(T128x128w8, 128, 128, 2, 4)
        W4A8_TILE(T256x128, 256, 128, 2, 2)
        W4A8_TILE(T256x128w8, 256, 128, 4, 2)
        W4A8_TILE(T256x160, 256, 160, 4, 1)
        W4A8_TILE(T128x160, 128, 160, 4, 1)
    case TileShape::T256x320w8:
    case TileShape::TSkinny:
    case TileShape::TRows:
        return -1;
    }
#undef W4A8_TILE
    return -1;
}

template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS> struct LaunchCfgF {
    static int run(const GemmArgs &a, hipStream_t st)
    {
        launch_cfg<BM, BN, WM, WN, MODE, GS>(a, st);
        return 0;
    }
};
template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS> struct OccF {
    static int run() { return groups_per_cu<BM, BN, WM, WN, MODE, GS>(); }
};

template <GemmMode MODE, int GS>
void launch_mode(const GemmArgs &a, hipStream_t st)
{
    const TileShape t = choose_tile(MODE, GS, a.M, a.N, a.K, a.num_cu);
    if (t == TileShape::T256x320w8)
        launch_gemm_pc2(MODE == GemmMode::I32, a, st, true);
    else if (t == TileShape::TSkinny)
        launch_gemm_skinny(MODE == GemmMode::I32, a, st, true);
    else if (t == TileShape::TRows)
        launch_gemm_rows(MODE == GemmMode::I32, a, st, true);
    else
        with_tile<MODE, GS, LaunchCfgF>(t, a, st);
}

template <GemmMode MODE, int GS>
int resident_groups(TileShape t)
{
    const int o = with_tile<MODE, GS, OccF>(t);
    return o > 0 ? o : 1;
}

template <GemmMode MODE, int GS>
TileInfo info_mode(const GemmArgs &a)
{
    const TileShape t = choose_tile(MODE, GS, a.M, a.N, a.K, a.num_cu);
    if (t == TileShape::T256x320w8)
        return launch_gemm_pc2(MODE == GemmMode::I32, a, nullptr, false);
    if (t == TileShape::TSkinny)
        return launch_gemm_skinny(MODE == GemmMode::I32, a, nullptr, false);
    if (t == TileShape::TRows)
        return launch_gemm_rows(MODE == GemmMode::I32, a, nullptr, false);
    TileInfo r = tile_dims(t);
    const int64_t tiles = (int64_t)((a.M + r.bm - 1) / r.bm) * ((a.N + r.bn - 1) / r.bn);
    r.per_cu = resident_groups<MODE, GS>(t);
    const int64_t resident = (int64_t)a.num_cu * r.per_cu;
    r.tiles = tiles;
    r.grid = tiles < resident ? tiles : resident;
    return r;
}

}  // namespace

// Pick a tile shape: large tiles when the output is big, smaller ones when
// too few tiles would leave compute units idle.  The per-group modes hold
// fp32 accumulators next to the int32 ones, so their large tile is 256x128
// with eight 64x64 waves (two per SIMD, which lets one wave's fold run beside
// the other's MFMAs) rather than four larger ones.  Each raw-sum export takes
// exactly the tile of the product it checks (I32 that of PC, the partials
// that of their per-group product).
TileShape choose_tile(GemmMode mode, int gs, int M, int N, int K, int num_cu)
{
    const bool pergroup = mode != GemmMode::PC && mode != GemmMode::I32;
    const bool int4 = mode == GemmMode::W4 || mode == GemmMode::W4_PARTIALS;
    const bool pg64 = (mode == GemmMode::PG || mode == GemmMode::PG_PARTIALS) && gs == 64;
    const int64_t t256x160 = (int64_t)((M + 255) / 256) * ((N + 159) / 160);
    const int64_t t256x128 = (int64_t)((M + 255) / 256) * ((N + 127) / 128);
    const int64_t t128x128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    // Tens to hundreds of tokens per channel: the product is bound by moving
    // bytes.  The row-range form with shared stages (one compute unit per
    // weight-row range and token slice) measured faster than the tiles for
    // 33-256 tokens wherever it applies (K % 128 == 0), warm and with the
    // weights from HBM (warm / cold us against the tiles: 64x10240x2560
    // 7.7 / 8.8 against 9.3 / 10.4, 128x10240x2560 9.7 / 10.3 against
    // 9.9 / 13.2, 256x10240x2560 13.1 / 16.3 against 13.9 / 21.8,
    // 128x14336x4096 15.3 / 19.6 against 15.9 / 20.4, 256x4096x14336 29.2
    // against 39).
    if (!pergroup && M > 32 && M <= 256 && plan_gemm_rows(M, N, K, num_cu).ok)
        return TileShape::TRows;
    // Few tokens per channel: the product is bound by one pass over the
    // weights, and the row-range form that splits K over its waves (each
    // compute unit streams a range of weight rows against all tokens)
    // measured faster up to 32 tokens, and up to 128 where the output is too
    // narrow (N <= 8192) for enough tiles and K % 128 != 0.  Every compute
    // unit reads all of X, so beyond that the tiles win.
    if (!pergroup && (M <= 32 || (M <= 128 && N <= 8192)))
        return TileShape::TSkinny;
    // Few tokens: the weights are streamed once and the output is small, so
    // the tile count decides how many compute units pull weights.  32x32
    // single-wave tiles (int8 weights) and 64x64 ones (per-channel) give four
    // and two times the tiles of 32x128 / 64x128; the narrow tiles did not pay
    // for W4A8, nor for the per-group modes above 32 tokens.
    if (M <= 32)
        return int4 ? TileShape::T32x128 : TileShape::T32x32;
    if (M <= 64)
        return pergroup ? TileShape::T64x128 : TileShape::T64x64;
    if (!pergroup) {
        // Large outputs: the cheapest of the big tiles by (rounds of tiles
        // over the compute units) x (tile area / its measured relative rate:
        // 256x320 1.08, 256x160 1, 256x128 0.9, 128x128 0.85, 128x160 0.8),
        // so that a last round left mostly empty counts against a tile shape
        // (128x160 fills the compute units where the 256-row tiles leave
        // many idle, e.g. 4096 x 1280).  The 256x320 kernel needs
        // K % 128 == 0.
        if (t128x128 >= 256) {
            const int64_t cu = num_cu > 0 ? num_cu : 1;
            const int64_t t256x320 = (int64_t)((M + 255) / 256) * ((N + 319) / 320);
            auto rounds = [&](int64_t t) { return (double)((t + cu - 1) / cu); };
            const double c320 = (N % 320 == 0 && K % 128 == 0)
                                    ? rounds(t256x320) * (256.0 * 320.0 / 1.08) : 1e300;
            const double c160 = N % 160 == 0 ? rounds(t256x160) * (256.0 * 160.0) : 1e300;
            const double c256 = rounds(t256x128) * (256.0 * 128.0 / 0.9);
            const double c128 = rounds(t128x128) * (128.0 * 128.0 / 0.85);
            const int64_t t128x160 = (int64_t)((M + 127) / 128) * ((N + 159) / 160);
            const double c160h = N % 160 == 0 ? rounds(t128x160) * (128.0 * 160.0 / 0.8) : 1e300;
            const double best = std::min(std::min(c320, c160), std::min(std::min(c256, c128), c160h));
            if (c320 == best)
                return TileShape::T256x320w8;
            if (c160 == best)
                return TileShape::T256x160;
            if (c160h == best)
                return TileShape::T128x160;
            if (c256 == best)
                return TileShape::T256x128;
            return TileShape::T128x128;
        }
    }
    // per-group gs=64 at 256x128 needs more than the 256 registers a wave
    // has at two waves per SIMD (it spills); it takes 128x128 below
    if (pergroup && !pg64 && t256x128 >= 384)
        return TileShape::T256x128w8;   // two waves per SIMD: folds run beside MFMAs
    // per-group gs=64 is bound by its fold (VALU): eight 64x32 waves (two per
    // SIMD, few registers) overlap one wave's fold with another's MFMAs; the
    // extra LDS reads of the narrower waves cost nothing at its MFMA rate
    if (pg64 && t128x128 >= 256)
        return TileShape::T128x128w8;
    return t128x128 >= 256 ? TileShape::T128x128 : TileShape::T64x128;
}

TileInfo tile_dims(TileShape t)
{
    TileInfo r{};
    switch (t) {
    case TileShape::T32x32: r.bm = 32; r.bn = 32; r.waves = 1; break;
    case TileShape::T32x128: r.bm = 32; r.bn = 128; r.waves = 4; break;
    case TileShape::T64x64: r.bm = 64; r.bn = 64; r.waves = 2; break;
    case TileShape::T64x128: r.bm = 64; r.bn = 128; r.waves = 4; break;
    case TileShape::T128x128: r.bm = 128; r.bn = 128; r.waves = 4; break;
    case TileShape::T128x128w8: r.bm = 128; r.bn = 128; r.waves = 8; break;
    case TileShape::T256x128: r.bm = 256; r.bn = 128; r.waves = 4; break;
    case TileShape::T256x128w8: r.bm = 256; r.bn = 128; r.waves = 8; break;
    case TileShape::T256x160: r.bm = 256; r.bn = 160; r.waves = 4; break;
    case TileShape::T128x160: r.bm = 128; r.bn = 160; r.waves = 4; break;
    case TileShape::T256x320w8: r.bm = 256; r.bn = 320; r.waves = 8; break;
    case TileShape::TSkinny: r.bm = 0; r.bn = 0; r.waves = 4; break;   // depends on M and N
    case TileShape::TRows: r.bm = 0; r.bn = 0; r.waves = 4; break;     // depends on M and N
    }
    return r;
}

namespace {

// Dispatch on the mode and group size (template arguments).
template <template <GemmMode, int> class F, typename... A>
auto by_mode(GemmMode mode, int gs, A &&...args)
{
    switch (mode) {
    case GemmMode::PC: return F<GemmMode::PC, 0>::run(args...);
    case GemmMode::I32: return F<GemmMode::I32, 0>::run(args...);
    case GemmMode::PG:
        return gs == 64 ? F<GemmMode::PG, 64>::run(args...) : F<GemmMode::PG, 128>::run(args...);
    case GemmMode::PG_PARTIALS:
        return gs == 64 ? F<GemmMode::PG_PARTIALS, 64>::run(args...)
                        : F<GemmMode::PG_PARTIALS, 128>::run(args...);
    case GemmMode::W4:
        return gs == 64 ? F<GemmMode::W4, 64>::run(args...) : F<GemmMode::W4, 128>::run(args...);
    case GemmMode::W4_PARTIALS:
        return gs == 64 ? F<GemmMode::W4_PARTIALS, 64>::run(args...)
                        : F<GemmMode::W4_PARTIALS, 128>::run(args...);
    }
    return F<GemmMode::PC, 0>::run(args...);
}

template <GemmMode MODE, int GS> struct LaunchF {
    static int run(const GemmArgs &a, hipStream_t st)
    {
        launch_mode<MODE, GS>(a, st);
        return 0;
    }
};
template <GemmMode MODE, int GS> struct InfoF {
    static TileInfo run(const GemmArgs &a) { return info_mode<MODE, GS>(a); }
};

}  // namespace

TileInfo gemm_info(GemmMode mode, const GemmArgs &a)
{
    return by_mode<InfoF>(mode, a.gs, a);
}

void launch_gemm(GemmMode mode, const GemmArgs &a, hipStream_t st)
{
    by_mode<LaunchF>(mode, a.gs, a, st);
}

}  // namespace w4a8
