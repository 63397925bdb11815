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
// Design (CDNA4, wave64, one wave per SIMD for the large tiles):
//  * One workgroup computes a BM x BN tile of Y (m x n) with WM x WN waves.
//    Both operands are K-contiguous.  v_mfma_i32_32x32x32_i8 takes the
//    weight fragment as its A operand (32 n-rows x 32 k, 16 bytes per lane)
//    and the activation fragment as B, so each lane's int32 results come in
//    runs of four consecutive n of one output row (8-byte fp16 stores).  This
//    MFMA sustains close to the int8 peak with a single wave per SIMD, which
//    the large per-wave tiles need (they keep LDS traffic per op low).
//  * K advances in stages of 128 bytes through three LDS buffers.  Global
//    loads for stages s+2 and s+3 are in flight in two register sets while
//    stage s is computed; stage s+2 is written to LDS at the end of stage s,
//    so stage s+1 is already resident when stage s ends and its first
//    fragments are read while the last MFMAs of stage s run.  Within a stage
//    the fragments of k-step t+1 are read while the MFMAs of step t run.
//  * 16-byte chunks are XOR-swizzled per LDS row.
//  * int4 weights are loaded packed (half the bytes), unpacked in registers to
//    16 * code (the nibble placed in the high half of each byte, which is
//    the code times 16 as a signed byte) and stored to LDS in the same int8
//    layout; the factor 16 is folded into the weight scales (exact).
//  * Per-group modes restart the int32 accumulators for every group and fold
//    them into fp32 accumulators with the group's scales, which are staged
//    through LDS together with the tiles.
//  * Workgroups are remapped so that each XCD (one L2 each) works on a
//    contiguous range of tiles, ordered in groups of `group_m` tile rows.
#include <type_traits>

#include "kernels.hpp"

namespace w4a8 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 128;          // k bytes per LDS stage (four 32-wide MFMA steps)

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

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

// Workgroup barrier that orders LDS accesses only: global loads stay in
// flight across it (a full __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <GemmMode MODE> struct ModeTraits {
    static constexpr bool int4 = (MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool pergroup = (MODE == GemmMode::PG || MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool partials = (MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4_PARTIALS);
    static constexpr bool fold_sa = (MODE == GemmMode::PG);     // per-group activation scales
    static constexpr bool fold_sw = (MODE == GemmMode::PG || MODE == GemmMode::W4);
};

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS copies: each lane's bytes from global memory land at
// M0 + size * lane.  Issued through asm so that the only waits on them are
// the kernel's own (vmcnt before the barrier that publishes a stage); the
// "memory" clobber keeps other memory accesses from moving across them.  M0
// is saved and restored around the copy, and one wait state separates the
// SALU write of M0 from the load that reads it (a gfx9 hazard).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(src)
                 : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const void *src, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(src)
                 : "memory");
}

// s_waitcnt that waits for the vector-memory counter only (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maximum).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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
    // copies every wave issues per stage (a lower bound where the scale
    // instructions do not split evenly; waiting on it is conservative)
    constexpr int ND = XB + WB + SA_I / NW + SW_I / NW;

    __shared__ __attribute__((aligned(1024))) int8_t xs0[XBUF];
    __shared__ __attribute__((aligned(1024))) int8_t xs1[XBUF];
    __shared__ __attribute__((aligned(1024))) int8_t xs2[XBUF];
    __shared__ __attribute__((aligned(1024))) int8_t ws0[WBUF];
    __shared__ __attribute__((aligned(1024))) int8_t ws1[WBUF];
    __shared__ __attribute__((aligned(1024))) int8_t ws2[WBUF];
    constexpr int SAL = T::fold_sa ? NG * BM : 1, SWL = T::fold_sw ? NG * BN : 1;
    __shared__ __attribute__((aligned(16))) float sa0[SAL], sa1[SAL], sa2[SAL];
    __shared__ __attribute__((aligned(16))) float sw0[SWL], sw1[SWL], sw2[SWL];
    auto XS = [&](auto B) __attribute__((always_inline)) -> int8_t * {
        constexpr int b = decltype(B)::value;
        return b == 0 ? xs0 : (b == 1 ? xs1 : xs2);
    };
    auto WS = [&](auto B) __attribute__((always_inline)) -> int8_t * {
        constexpr int b = decltype(B)::value;
        return b == 0 ? ws0 : (b == 1 ? ws1 : ws2);
    };
    auto SAS = [&](auto B) __attribute__((always_inline)) -> float * {
        constexpr int b = decltype(B)::value;
        return b == 0 ? sa0 : (b == 1 ? sa1 : sa2);
    };
    auto SWS = [&](auto B) __attribute__((always_inline)) -> float * {
        constexpr int b = decltype(B)::value;
        return b == 0 ? sw0 : (b == 1 ? sw1 : sw2);
    };

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile selection: XCD-contiguous ranges, grouped along m
    int tm, tn;
    {
        const int nb = (int)gridDim.x, bid = (int)blockIdx.x;
        const int xcd = bid & 7, local = bid >> 3;
        const int per = nb >> 3, rem = nb & 7;
        const int lid = (xcd < rem) ? xcd * (per + 1) + local
                                    : rem * (per + 1) + (xcd - rem) * per + local;
        const int span = group_m * tiles_n;
        const int first_m = (lid / span) * group_m;
        const int gm = min(tiles_m - first_m, group_m);
        const int in = lid % span;
        tm = first_m + in % gm;
        tn = in / gm;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int G = T::pergroup ? K / GS : 1;
    const int nstage = (K + BK - 1) / BK;
    const int nks = K / 32;                           // 32-wide MFMA steps in K

    const int8_t *__restrict__ xq = args.xq;
    const uint8_t *__restrict__ wb = static_cast<const uint8_t *>(args.w);
    const int wrow = T::int4 ? K / 2 : K;             // bytes per weight row

    // Direct-to-LDS source offsets.  A wave instruction writes lane l's 16
    // bytes at LDS block + 16*l, i.e. row 8*blk + l/8, physical chunk l%8; the
    // lane therefore fetches the logical chunk that the swizzle puts there.
    const int dma_row = lane >> 3;
    const int dma_chunk = (lane & 7) ^ (dma_row & 7);
    int64_t xoff[XB];
#pragma unroll
    for (int i = 0; i < XB; ++i) {
        const int row = (wave + NW * i) * 8 + dma_row;
        xoff[i] = (int64_t)min(m0 + row, M - 1) * K + dma_chunk * 16;
    }
    int64_t woff[WB > 0 ? WB : 1];
#pragma unroll
    for (int i = 0; i < WB; ++i) {
        const int row = (wave + NW * i) * 8 + dma_row;
        woff[i] = (int64_t)min(n0 + row, N - 1) * K + dma_chunk * 16;
    }
    // packed int4 weights: thread -> (row, 16-byte packed chunk)
    int64_t w4off[WIT4 > 0 ? WIT4 : 1];
#pragma unroll
    for (int it = 0; it < WIT4; ++it) {
        const int q = min(tid + it * NW * 64, WCH4 - 1);
        w4off[it] = (int64_t)min(n0 + (q >> 2), N - 1) * wrow + (q & 3) * 16;
    }

    // Issue the copies of stage s into LDS buffer B.
    auto dma_stage = [&](auto B, int s) __attribute__((always_inline)) {
        const int k0 = s * BK;
        const bool full = k0 + BK <= K;               // else: K % 128 == 64, upper half unused
        const int kx = (full || k0 + dma_chunk * 16 < K) ? k0 : K - 16 - dma_chunk * 16;
#pragma unroll
        for (int i = 0; i < XB; ++i)
            copy16_to_lds(xq + xoff[i] + kx, lds_addr(XS(B) + (wave + NW * i) * 1024));
#pragma unroll
        for (int i = 0; i < WB; ++i)
            copy16_to_lds(wb + woff[i] + kx, lds_addr(WS(B) + (wave + NW * i) * 1024));
        if constexpr (T::fold_sa) {
#pragma unroll
            for (int i = 0; i < (SA_I + NW - 1) / NW; ++i) {
                const int ins = wave + NW * i;
                if (SA_I % NW == 0 || ins < SA_I) {
                    const int e = ins * 64 + lane;    // entry g*BM + r
                    const int g = min(e / BM, NG - 1), r = e % BM;
                    const int gi = min(s * NG + g, G - 1);
                    if (e < NG * BM)
                        copy4_to_lds(args.sa + (int64_t)min(m0 + r, M - 1) * G + gi,
                                     lds_addr(SAS(B) + ins * 64));
                }
            }
        }
        if constexpr (T::fold_sw) {
#pragma unroll
            for (int i = 0; i < (SW_I + NW - 1) / NW; ++i) {
                const int ins = wave + NW * i;
                if (SW_I % NW == 0 || ins < SW_I) {
                    const int e = ins * 64 + lane;    // entry g*BN + r
                    const int g = min(e / BN, NG - 1), r = e % BN;
                    const int gi = min(s * NG + g, G - 1);
                    if (e < NG * BN)
                        copy4_to_lds(args.sw + (int64_t)min(n0 + r, N - 1) * G + gi,
                                     lds_addr(SWS(B) + ins * 64));
                }
            }
        }
    };

    // ---- packed int4 weights: register staging and unpack into LDS
    uint4 w4r[WIT4 > 0 ? WIT4 : 1];
    auto w4_load = [&](int s) __attribute__((always_inline)) {
        const int kb0 = s * (BK / 2);
#pragma unroll
        for (int it = 0; it < WIT4; ++it) {
            const int c = (tid + it * NW * 64) & 3;
            const bool ok = kb0 + c * 16 < wrow;
            w4r[it] = *reinterpret_cast<const uint4 *>(wb + w4off[it] + (ok ? kb0 : wrow - 16 - c * 16));
        }
    };
    auto w4_store = [&](auto B) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < WIT4; ++it) {
            const int q = tid + it * NW * 64;
            if (WCH4 % (NW * 64) == 0 || q < WCH4) {
                const int row = q >> 2, c = q & 3;    // packed chunk c -> int8 chunks 2c, 2c+1
                const uint2 a = unpack_int4x8(w4r[it].x), b = unpack_int4x8(w4r[it].y);
                const uint2 d = unpack_int4x8(w4r[it].z), e = unpack_int4x8(w4r[it].w);
                *reinterpret_cast<uint4 *>(WS(B) + row * BK + swz(row, 2 * c) * 16) =
                    make_uint4(a.x, a.y, b.x, b.y);
                *reinterpret_cast<uint4 *>(WS(B) + row * BK + swz(row, 2 * c + 1) * 16) =
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
    if constexpr (T::fold_sw) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                accf[j][i] = v16f{};
    }

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
    // output coordinates of this lane inside a 32x32 block: m = lane%32,
    // n = 8*(r/4) + 4*(lane/32) + r%4 for accumulator element r
    const int out_m = lane & 31;
    const int out_n = lhalf * 4;

    struct Frag {
        v4i a[FN];    // weights (A operand)
        v4i b[FM];    // activations (B operand)
    };
    Frag f0, f1;

    auto read_frag = [&](Frag &F, auto B, int t) __attribute__((always_inline)) {
        const int8_t *xb = XS(B) + xrow0 * BK + fo[t];
        const int8_t *wbf = WS(B) + wrow0 * BK + fo[t];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            F.b[i] = *reinterpret_cast<const v4i *>(xb + i * 32 * BK);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            F.a[j] = *reinterpret_cast<const v4i *>(wbf + j * 32 * BK);
    };

    auto mfma_step = [&](const Frag &F, bool restart) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.a[j], F.b[i],
                                                                  restart ? v16i{} : acc[j][i], 0, 0, 0);
    };

    auto store_partials = [&](int g) __attribute__((always_inline)) {
        int32_t *P = static_cast<int32_t *>(args.out) + (int64_t)g * M * N;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 32 + out_m;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * TN + j * 32 + q * 8 + out_n;
                    v4i v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                             acc[j][i][4 * q + 3]};
                    if constexpr (T::int4)
                        v = v >> 4;                       // exact: the sums are 16 * P
                    int32_t *dst = P + (int64_t)m * N + n;
                    if (n + 3 < N && (N & 3) == 0) {
                        *reinterpret_cast<v4i *>(dst) = v;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                dst[r] = v[r];
                    }
                }
        }
    };

    auto fold_group = [&](auto B, int g) __attribute__((always_inline)) {
        float sav[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            sav[i] = T::fold_sa ? SAS(B)[g * BM + wm * TM + i * 32 + out_m] : 1.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f swv = *reinterpret_cast<const v4f *>(
                    &SWS(B)[g * BN + wn * TN + j * 32 + q * 8 + out_n]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sc = T::fold_sa ? sav[i] * swv[r] : swv[r];
                        accf[j][i][4 * q + r] =
                            fmaf((float)acc[j][i][4 * q + r], sc, accf[j][i][4 * q + r]);
                    }
            }
    };

    // After k-step t of stage s: close a group if one ends here.
    auto after_step = [&](auto B, int s, int t) __attribute__((always_inline)) {
        if constexpr (T::pergroup) {
            const int ks = s * 4 + t;
            if ((t + 1) % SPG == 0 || ks + 1 == nks) {
                const int gl = t / SPG;                   // group slot within the stage
                if constexpr (T::partials)
                    store_partials(s * NG + gl);
                else
                    fold_group(B, gl);
            }
        }
    };

    // ---- pipeline.  Stage t lives in LDS buffer t % 3.  Its copies are
    // issued during step 3 of iteration t-3 (int4 weights: loaded into
    // registers in iteration t-2 and unpacked to LDS before the barrier of
    // iteration t-1).  Iteration s: steps 0-2 from buffer s%3; wait for
    // stage s+1's copies and barrier; issue stage s+3's copies into buffer
    // s%3 (nobody reads it any more); step 3, which also reads the first
    // fragments of stage s+1.  Every iteration issues the same memory
    // operations -- past the last stage the copies repeat the last stage
    // into a buffer nobody reads -- so the loop has no branches around them
    // and every wait count is a constant.
    const int last = nstage - 1;
    auto main_loop = [&](auto KFULL) __attribute__((always_inline)) {
        constexpr bool kfull = decltype(KFULL)::value;   // K % 128 == 0: every k-step exists
        dma_stage(std::integral_constant<int, 0>(), 0);
        if constexpr (T::int4) {
            w4_load(0);
            w4_store(std::integral_constant<int, 0>());
            w4_load(min(1, last));
        }
        dma_stage(std::integral_constant<int, 1>(), min(1, last));
        dma_stage(std::integral_constant<int, 2>(), min(2, last));
        wait_vmcnt<2 * ND>();
        lds_barrier();
        read_frag(f0, std::integral_constant<int, 0>(), 0);

        auto iteration = [&](auto B, int s) __attribute__((always_inline)) {
            constexpr int b = decltype(B)::value;
            constexpr int b1 = (b + 1) % 3;
            const int ks0 = s * 4;
            auto step = [&](auto TC) __attribute__((always_inline)) {
                constexpr int t = decltype(TC)::value;
                Frag &cur = (t & 1) ? f1 : f0;
                Frag &nxt = (t & 1) ? f0 : f1;
                if (kfull || ks0 + t < nks) {
                    if constexpr (t < 3) {
                        if (kfull || ks0 + t + 1 < nks)
                            read_frag(nxt, B, t + 1);
                    } else {
                        read_frag(nxt, std::integral_constant<int, b1>(), 0);
                    }
                    // keep the reads for the next step ahead of this step's
                    // MFMAs, which use fragments read one step earlier
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_step(cur, T::pergroup && (t % SPG == 0));
                    __builtin_amdgcn_sched_barrier(0);
                    after_step(B, s, t);
                }
            };
            step(std::integral_constant<int, 0>());
            step(std::integral_constant<int, 1>());
            step(std::integral_constant<int, 2>());
            // stage s+1 complete and visible; buffer b free
            if constexpr (T::int4)
                w4_store(std::integral_constant<int, b1>());
            wait_vmcnt<ND>();
            lds_barrier();
            if constexpr (T::int4)
                w4_load(min(s + 2, last));
            if constexpr (T::fold_sw) {
                // the fold after step 3 still reads this stage's scales from
                // buffer b: copy into it only afterwards
                step(std::integral_constant<int, 3>());
                dma_stage(B, min(s + 3, last));
            } else {
                dma_stage(B, min(s + 3, last));
                step(std::integral_constant<int, 3>());
            }
        };
        for (int s = 0; s < nstage; s += 3) {
            iteration(std::integral_constant<int, 0>(), s);
            if (s + 1 < nstage) {
                iteration(std::integral_constant<int, 1>(), s + 1);
                if (s + 2 < nstage)
                    iteration(std::integral_constant<int, 2>(), s + 2);
            }
        }
        // no copy may still be writing LDS when the workgroup ends
        wait_vmcnt<0>();
    };
    if (K % BK == 0)
        main_loop(std::true_type());
    else
        main_loop(std::false_type());

    // ---- epilogue
    if constexpr (T::partials) {
        return;
    } else if constexpr (MODE == GemmMode::I32) {
        int32_t *C = static_cast<int32_t *>(args.out);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 32 + out_m;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * TN + j * 32 + q * 8 + out_n;
                    const v4i v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                                   acc[j][i][4 * q + 3]};
                    int32_t *dst = C + (int64_t)m * N + n;
                    if (n + 3 < N && (N & 3) == 0) {
                        *reinterpret_cast<v4i *>(dst) = v;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                dst[r] = v[r];
                    }
                }
        }
    } else {
        uint16_t *Y = static_cast<uint16_t *>(args.out);
        const bool vec_ok = (N & 3) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 32 + out_m;
            if (m >= M)
                continue;
            const float sa = (MODE == GemmMode::PG) ? 1.0f : args.sa[m];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * TN + j * 32 + q * 8 + out_n;
                    float v[4];
                    if constexpr (MODE == GemmMode::PC) {
                        float swq[4];
                        if (vec_ok && n + 3 < N) {
                            const float4 t4 = *reinterpret_cast<const float4 *>(args.sw + n);
                            swq[0] = t4.x; swq[1] = t4.y; swq[2] = t4.z; swq[3] = t4.w;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                swq[r] = args.sw[min(n + r, N - 1)];
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = rescale_pc(acc[j][i][4 * q + r], sa, swq[r]);
                    } else if constexpr (MODE == GemmMode::PG) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = accf[j][i][4 * q + r];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = accf[j][i][4 * q + r] * (sa * 0.0625f);   // W4: per-token scale, undo x16 (exact)
                    }
                    uint16_t *dst = Y + (int64_t)m * N + n;
                    if (vec_ok && n + 3 < N) {
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_h2(v[0], v[1]),
                                                                     pack_h2(v[2], v[3]));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                dst[r] = f2h(v[r]);
                    }
                }
        }
    }
}

template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS>
void launch_cfg(const GemmArgs &a, hipStream_t st)
{
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int group_m = 4;
    const unsigned nb = (unsigned)tiles_m * (unsigned)tiles_n;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, GS>), dim3(nb), dim3(WM * WN * 64), 0, st,
                       a, tiles_m, tiles_n, group_m);
}

// Pick a tile shape: large tiles when the output is big, smaller ones when
// too few tiles would leave compute units idle.  The per-group modes hold
// fp32 accumulators next to the int32 ones and stay at 128x128 or below.
template <GemmMode MODE, int GS>
void launch_mode(const GemmArgs &a, hipStream_t st)
{
    constexpr bool pergroup = ModeTraits<MODE>::pergroup;
    const int64_t t256x160 = (int64_t)((a.M + 255) / 256) * ((a.N + 159) / 160);
    const int64_t t256x128 = (int64_t)((a.M + 255) / 256) * ((a.N + 127) / 128);
    const int64_t t128x128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (a.M <= 32) {
        launch_cfg<32, 128, 1, 4, MODE, GS>(a, st);
        return;
    }
    if (a.M <= 64) {
        launch_cfg<64, 128, 2, 2, MODE, GS>(a, st);
        return;
    }
    if constexpr (!pergroup) {
        if (t256x160 >= 512 && a.N % 160 == 0) {
            launch_cfg<256, 160, 4, 1, MODE, GS>(a, st);
            return;
        }
        if (t256x128 >= 512) {
            launch_cfg<256, 128, 2, 2, MODE, GS>(a, st);
            return;
        }
    }
    if (t128x128 >= 256)
        launch_cfg<128, 128, 2, 2, MODE, GS>(a, st);
    else
        launch_cfg<64, 128, 2, 2, MODE, GS>(a, st);
}

}  // namespace

void launch_gemm(GemmMode mode, const GemmArgs &a, hipStream_t st)
{
    switch (mode) {
    case GemmMode::PC: launch_mode<GemmMode::PC, 0>(a, st); break;
    case GemmMode::I32: launch_mode<GemmMode::I32, 0>(a, st); break;
    case GemmMode::PG:
        if (a.gs == 64) launch_mode<GemmMode::PG, 64>(a, st);
        else launch_mode<GemmMode::PG, 128>(a, st);
        break;
    case GemmMode::PG_PARTIALS:
        if (a.gs == 64) launch_mode<GemmMode::PG_PARTIALS, 64>(a, st);
        else launch_mode<GemmMode::PG_PARTIALS, 128>(a, st);
        break;
    case GemmMode::W4:
        if (a.gs == 64) launch_mode<GemmMode::W4, 64>(a, st);
        else launch_mode<GemmMode::W4, 128>(a, st);
        break;
    case GemmMode::W4_PARTIALS:
        if (a.gs == 64) launch_mode<GemmMode::W4_PARTIALS, 64>(a, st);
        else launch_mode<GemmMode::W4_PARTIALS, 128>(a, st);
        break;
    }
}

}  // namespace w4a8
