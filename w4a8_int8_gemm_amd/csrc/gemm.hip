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
// Design (CDNA4, wave64):
//  * One workgroup computes a BM x BN tile of Y (m x n) with WM x WN waves.
//    Both operands are K-contiguous, the natural layout for MFMA: the weight
//    tile feeds the MFMA's A operand (16 n-rows x 64 k per
//    v_mfma_i32_16x16x64_i8) and the activation tile its B operand, so each
//    lane's four int32 results are four consecutive n of one output row and
//    the epilogue stores 8 contiguous bytes per lane.
//  * K advances in stages of 128 bytes.  Global loads for stage s+1 are
//    issued into registers before the MFMAs of stage s, then written to the
//    other half of a double-buffered LDS tile.  16-byte chunks are XOR-
//    swizzled per row so that the ds_read_b128 fragment loads hit distinct
//    banks with either 32 or 64 four-byte banks.
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

constexpr int BK = 128;          // k bytes per LDS stage (two 64-wide MFMA steps)

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

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

template <GemmMode MODE> struct ModeTraits {
    static constexpr bool int4 = (MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool pergroup = (MODE == GemmMode::PG || MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4 || MODE == GemmMode::W4_PARTIALS);
    static constexpr bool partials = (MODE == GemmMode::PG_PARTIALS ||
                                      MODE == GemmMode::W4_PARTIALS);
    static constexpr bool fold_sa = (MODE == GemmMode::PG);     // per-group activation scales
    static constexpr bool fold_sw = (MODE == GemmMode::PG || MODE == GemmMode::W4);
};

// Workgroup barrier that orders LDS accesses only: global loads stay in
// flight across it (a full __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int BM, int BN, int WM, int WN, GemmMode MODE, int GS>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(GemmArgs args, int tiles_m,
                                                           int tiles_n, int group_m)
{
    using T = ModeTraits<MODE>;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    constexpr int XCH = BM * 8;                       // 16-byte chunks of X per stage
    constexpr int CPR = T::int4 ? 4 : 8;              // loaded 16-byte chunks per W row per stage
    constexpr int WCH = BN * CPR;
    constexpr int XIT = (XCH + NT - 1) / NT;
    constexpr int WIT = (WCH + NT - 1) / NT;
    // groups per stage (gs 64: two, gs 128: one); scales staged per group
    constexpr int NG = (GS == 64) ? 2 : 1;

    __shared__ __attribute__((aligned(16))) int8_t xs[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t ws[2][BN * BK];
    __shared__ __attribute__((aligned(16))) float sas[2][T::fold_sa ? NG * BM : 1];
    __shared__ __attribute__((aligned(16))) float sws[2][T::fold_sw ? NG * BN : 1];

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const int nkc = K / 64;                           // 64-wide MFMA steps in K

    const int8_t *__restrict__ xq = args.xq;
    const uint8_t *__restrict__ wb = static_cast<const uint8_t *>(args.w);
    const int wrow = T::int4 ? K / 2 : K;             // bytes per weight row

    // Per-thread global source offsets of its chunks (row clamped to the
    // matrix, so edge tiles read valid memory; those rows are never stored).
    int64_t xoff[XIT], woff[WIT];
#pragma unroll
    for (int it = 0; it < XIT; ++it) {
        const int q = min(tid + it * NT, XCH - 1);
        xoff[it] = (int64_t)min(m0 + (q >> 3), M - 1) * K + (q & 7) * 16;
    }
#pragma unroll
    for (int it = 0; it < WIT; ++it) {
        const int q = min(tid + it * NT, WCH - 1);
        woff[it] = (int64_t)min(n0 + q / CPR, N - 1) * wrow + (q % CPR) * 16;
    }

    // ---- register staging: two stages in flight
    struct Stage {
        uint4 x[XIT];
        uint4 w[WIT];
        float sa[NG];
        float sw[NG];
    };
    Stage st0;
    [[maybe_unused]] Stage st1;

    auto load_stage = [&](Stage &S, int s) {
        const int k0 = s * BK;
        const int kb0 = T::int4 ? k0 / 2 : k0;
        if (k0 + BK <= K) {
#pragma unroll
            for (int it = 0; it < XIT; ++it)
                S.x[it] = *reinterpret_cast<const uint4 *>(xq + xoff[it] + k0);
#pragma unroll
            for (int it = 0; it < WIT; ++it)
                S.w[it] = *reinterpret_cast<const uint4 *>(wb + woff[it] + kb0);
        } else {
            // last stage of a K with K % 128 == 64: the upper half is zero
#pragma unroll
            for (int it = 0; it < XIT; ++it) {
                const int c = (tid + it * NT) & 7;
                const bool ok = k0 + c * 16 < K;
                const uint4 v = *reinterpret_cast<const uint4 *>(xq + xoff[it] + (ok ? k0 : K - 16 - c * 16));
                S.x[it] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int it = 0; it < WIT; ++it) {
                const int c = (tid + it * NT) % CPR;
                const bool ok = kb0 + c * 16 < wrow;
                const uint4 v = *reinterpret_cast<const uint4 *>(wb + woff[it] + (ok ? kb0 : wrow - 16 - c * 16));
                S.w[it] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        if constexpr (T::fold_sa) {
            if (tid < BM) {
                const int gr = min(m0 + tid, M - 1);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int gi = min(s * NG + g, G - 1);
                    S.sa[g] = args.sa[(int64_t)gr * G + gi];
                }
            }
        }
        if constexpr (T::fold_sw) {
            if (tid < BN) {
                const int gr = min(n0 + tid, N - 1);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int gi = min(s * NG + g, G - 1);
                    float v = args.sw[(int64_t)gr * G + gi];
                    if constexpr (T::int4)
                        v *= 0.0625f;                 // undo the x16 of the unpacked codes (exact)
                    S.sw[g] = v;
                }
            }
        }
    };

    auto store_stage = [&](const Stage &S, int buf) {
#pragma unroll
        for (int it = 0; it < XIT; ++it) {
            const int q = tid + it * NT;
            if (XCH % NT == 0 || q < XCH) {
                const int row = q >> 3, c = q & 7;
                *reinterpret_cast<uint4 *>(&xs[buf][row * BK + swz(row, c) * 16]) = S.x[it];
            }
        }
#pragma unroll
        for (int it = 0; it < WIT; ++it) {
            const int q = tid + it * NT;
            if (WCH % NT == 0 || q < WCH) {
                if constexpr (T::int4) {
                    const int row = q >> 2, c = q & 3;    // packed chunk c -> int8 chunks 2c, 2c+1
                    const uint2 a = unpack_int4x8(S.w[it].x), b = unpack_int4x8(S.w[it].y);
                    const uint2 d = unpack_int4x8(S.w[it].z), e = unpack_int4x8(S.w[it].w);
                    *reinterpret_cast<uint4 *>(&ws[buf][row * BK + swz(row, 2 * c) * 16]) =
                        make_uint4(a.x, a.y, b.x, b.y);
                    *reinterpret_cast<uint4 *>(&ws[buf][row * BK + swz(row, 2 * c + 1) * 16]) =
                        make_uint4(d.x, d.y, e.x, e.y);
                } else {
                    const int row = q >> 3, c = q & 7;
                    *reinterpret_cast<uint4 *>(&ws[buf][row * BK + swz(row, c) * 16]) = S.w[it];
                }
            }
        }
        if constexpr (T::fold_sa) {
            if (tid < BM) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    sas[buf][g * BM + tid] = S.sa[g];
            }
        }
        if constexpr (T::fold_sw) {
            if (tid < BN) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    sws[buf][g * BN + tid] = S.sw[g];
            }
        }
    };

    // ---- accumulators
    v4i acc[FN][FM];
    v4f accf[T::fold_sw ? FN : 1][T::fold_sw ? FM : 1];
    const v4i zero = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
            acc[j][i] = zero;
    if constexpr (T::fold_sw) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                accf[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // fragment addressing: lane reads row (base + lane%16), logical chunk 4*kk + lane/16
    const int lrow = lane & 15;
    const int lchunk = lane >> 4;
    const int xrow0 = wm * TM + lrow;
    const int wrow0 = wn * TN + lrow;
    // output coordinates of this lane inside a 16x16 block
    const int out_m = lane & 15;
    const int out_n = (lane >> 4) * 4;
    // swizzled byte offsets of the lane's fragment chunk for kk = 0, 1 (the
    // swizzle depends on the row only through lane%16, since bases are multiples of 16)
    const int xo0 = xrow0 * BK + swz(lrow, lchunk) * 16;
    const int xo1 = xrow0 * BK + swz(lrow, 4 + lchunk) * 16;
    const int wo0 = wrow0 * BK + swz(lrow, lchunk) * 16;
    const int wo1 = wrow0 * BK + swz(lrow, 4 + lchunk) * 16;

    auto store_partials = [&](int g) {
        int32_t *P = static_cast<int32_t *>(args.out) + (int64_t)g * M * N;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 16 + out_m;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 16 + out_n;
                v4i v = acc[j][i];
                if constexpr (T::int4)
                    v = v >> 4;                           // exact: the sums are 16 * P
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

    auto fold_group = [&](int buf, int g) {
        float sav[FM];
        v4f swv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            sav[i] = T::fold_sa ? sas[buf][g * BM + wm * TM + i * 16 + out_m] : 1.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
            swv[j] = *reinterpret_cast<const v4f *>(&sws[buf][g * BN + wn * TN + j * 16 + out_n]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sc = T::fold_sa ? sav[i] * swv[j][r] : swv[j][r];
                    accf[j][i][r] = fmaf((float)acc[j][i][r], sc, accf[j][i][r]);
                }
    };

    // One 64-wide k step from LDS buffer `buf`.
    auto mma_step = [&](int buf, int kk, bool restart) {
        const int8_t *xb = xs[buf];
        const int8_t *wbuf = ws[buf];
        const int xo = kk ? xo1 : xo0, wo = kk ? wo1 : wo0;
        v4i bf[FM], af[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            bf[i] = *reinterpret_cast<const v4i *>(xb + xo + i * 16 * BK);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            af[j] = *reinterpret_cast<const v4i *>(wbuf + wo + j * 16 * BK);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[j], bf[i],
                                                                  restart ? zero : acc[j][i], 0, 0, 0);
    };

    auto compute_stage = [&](int buf, int s) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kc = s * 2 + kk;
            if (kc < nkc) {
                // per-group modes start every group from zero
                mma_step(buf, kk, T::pergroup && (GS == 64 || kk == 0));
                if constexpr (T::pergroup) {
                    if (GS == 64 || kk == 1 || kc + 1 == nkc) {
                        const int g = (GS == 64) ? kc : s;
                        if constexpr (T::partials)
                            store_partials(g);
                        else
                            fold_group(buf, (GS == 64) ? kk : 0);
                    }
                }
            }
        }
    };

    // ---- pipeline.  Stage s is computed from LDS buffer s&1.  Without fp32
    // accumulators (per-channel) two register sets keep the loads of stages
    // s+1 and s+2 in flight; the per-group modes, which hold fp32
    // accumulators too, keep one stage in flight to stay within registers.
    if constexpr (!T::pergroup) {
        load_stage(st0, 0);
        if (nstage > 1)
            load_stage(st1, 1);
        store_stage(st0, 0);
        lds_barrier();
        auto iteration = [&](auto P, int s) {
            constexpr int p = decltype(P)::value;
            Stage &cur = p == 0 ? st0 : st1;    // held stage s (already in LDS)
            Stage &nxt = p == 0 ? st1 : st0;    // holds stage s+1
            if (s + 2 < nstage)
                load_stage(cur, s + 2);
            compute_stage(p, s);
            if (s + 1 < nstage)
                store_stage(nxt, p ^ 1);
            lds_barrier();
        };
        for (int s = 0; s < nstage; s += 2) {
            iteration(std::integral_constant<int, 0>(), s);
            if (s + 1 < nstage)
                iteration(std::integral_constant<int, 1>(), s + 1);
        }
    } else {
        load_stage(st0, 0);
        store_stage(st0, 0);
        lds_barrier();
        for (int s = 0; s < nstage; ++s) {
            if (s + 1 < nstage)
                load_stage(st0, s + 1);
            compute_stage(s & 1, s);
            if (s + 1 < nstage)
                store_stage(st0, (s + 1) & 1);
            lds_barrier();
        }
    }

    // ---- epilogue
    if constexpr (T::partials) {
        return;
    } else if constexpr (MODE == GemmMode::I32) {
        int32_t *C = static_cast<int32_t *>(args.out);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 16 + out_m;
            if (m >= M)
                continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 16 + out_n;
                int32_t *dst = C + (int64_t)m * N + n;
                if (n + 3 < N && (N & 3) == 0) {
                    *reinterpret_cast<v4i *>(dst) = acc[j][i];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            dst[r] = acc[j][i][r];
                }
            }
        }
    } else {
        uint16_t *Y = static_cast<uint16_t *>(args.out);
        v4f swv[FN];
        if constexpr (MODE == GemmMode::PC) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 16 + out_n;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    swv[j][r] = args.sw[min(n + r, N - 1)];
            }
        }
        const bool vec_ok = (N & 3) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 16 + out_m;
            if (m >= M)
                continue;
            const float sa = (MODE == GemmMode::PG) ? 1.0f : args.sa[m];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 16 + out_n;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (MODE == GemmMode::PC)
                        v[r] = rescale_pc(acc[j][i][r], sa, swv[j][r]);
                    else if constexpr (MODE == GemmMode::PG)
                        v[r] = accf[j][i][r];
                    else
                        v[r] = accf[j][i][r] * sa;     // W4: per-token scale last
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
// too few tiles would leave compute units idle.
template <GemmMode MODE, int GS>
void launch_mode(const GemmArgs &a, hipStream_t st)
{
    constexpr bool wide_ok = !ModeTraits<MODE>::pergroup;   // 256x160 only without fp32 accumulators
    const int64_t t256x160 = (int64_t)((a.M + 255) / 256) * ((a.N + 159) / 160);
    const int64_t t256x128 = (int64_t)((a.M + 255) / 256) * ((a.N + 127) / 128);
    const int64_t t128x128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (a.M <= 64) {
        launch_cfg<64, 64, 1, 4, MODE, GS>(a, st);
        return;
    }
    if constexpr (wide_ok) {
        if (t256x160 >= 512 && a.N % 160 == 0) {
            launch_cfg<256, 160, 2, 2, MODE, GS>(a, st);
            return;
        }
    }
    if (t256x128 >= 512)
        launch_cfg<256, 128, 2, 2, MODE, GS>(a, st);
    else if (t128x128 >= 256)
        launch_cfg<128, 128, 2, 2, MODE, GS>(a, st);
    else
        launch_cfg<128, 64, 2, 2, MODE, GS>(a, st);
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
