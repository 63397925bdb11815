// Launchers of the library's kernels (host side).  Arguments are validated by
// the C entry points before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace w4a8 {

// Quantize `rows` fp16 rows of length K (K % 8 == 0) with slices of gs
// (0 = whole row, 64, 128).  q is int8 [rows, K], or packed uint8
// [rows, K/2] when int4; scale is fp32 [rows] or [rows, K/gs].
void launch_quantize_rows(const uint16_t *x, int64_t rows, int K, int gs, float qmax, void *q,
                          float *scale, bool int4, hipStream_t st);

// What the GEMM's epilogue does with the int32 sums.
enum class GemmMode : int {
    PC = 0,          // fp16 y = c * sa[m] * sw[n]
    I32 = 1,         // int32 c
    PG = 2,          // fp16 y = sum_g P_g * sa[m,g] * sw[n,g]
    PG_PARTIALS = 3, // int32 P [G, M, N]
    W4 = 4,          // fp16 y = sa[m] * sum_g P_g * sw[n,g]   (int4 weights)
    W4_PARTIALS = 5  // int32 P [G, M, N]                       (int4 weights)
};

struct GemmArgs {
    const int8_t *xq;     // [M, K]
    const float *sa;      // [M] or [M, G]
    const void *w;        // int8 [N, K] or packed int4 [N, K/2]
    const float *sw;      // [N] or [N, G]
    void *out;            // fp16 [M, N] or int32 [M, N] / [G, M, N]
    int M, N, K, gs;
    int num_cu;           // compute units of the device (sizes the persistent grid)
};

void launch_gemm(GemmMode mode, const GemmArgs &a, hipStream_t st);

// Tile configurations of the GEMM kernel (BM x BN per workgroup; "w8" = eight
// waves, i.e. two per SIMD, where the default is four).
enum class TileShape : int {
    T32x32, T32x128, T64x64, T64x128, T128x128, T128x128w8, T128x160, T256x128, T256x128w8,
    T256x160,
    T256x320w8,  // the per-channel kernel of its own (K % 128 == 0)
    TSkinny,     // per-channel, few tokens: weight rows per workgroup, K split over its waves
    TRows        // per-channel, tens to hundreds of tokens: weight rows per workgroup, shared stages
};
struct TileInfo {
    int bm, bn, waves;    // output tile per workgroup and its wavefronts
    int64_t tiles;        // tiles of the M x N output
    int64_t grid;         // workgroups launched (persistent: at most what fits at once)
    int per_cu;           // workgroups a compute unit holds at once
};
// The tile a GEMM of this mode and size runs with on a device of num_cu
// compute units (each raw-sum export takes its product's choice).
TileShape choose_tile(GemmMode mode, int gs, int M, int N, int K, int num_cu);
TileInfo tile_dims(TileShape t);
// The tile and grid launch_gemm would use for these arguments.
TileInfo gemm_info(GemmMode mode, const GemmArgs &a);

// The per-channel (or raw int32, i32_out) GEMM on 256 x 320 tiles of eight
// waves (K % 128 == 0); launches only when `launch`, and returns its tile and
// grid either way.
TileInfo launch_gemm_pc2(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch);

// The per-channel (or raw int32) GEMM for few tokens (M <= 128, K % 64 == 0):
// each workgroup streams a contiguous range of weight rows against all tokens.
// Its TileInfo gives bm = the tokens padded to 16, bn = the rows of one pass.
TileInfo launch_gemm_skinny(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch);

// The per-channel (or raw int32) GEMM for tens to hundreds of tokens
// (K % 128 == 0): one workgroup per compute unit streams a contiguous range of
// weight rows against one or two slices of the tokens, whose four waves share
// 128-byte K stages in a deep LDS ring.  plan_gemm_rows gives its split (ok is
// false where it does not apply: more than 128 tokens per slice or 128 rows
// per range); TileInfo gives bm = the tokens of a slice padded to 64, bn = the
// rows of a range padded to 16.
struct RowsPlan {
    bool ok;
    int pm;       // token slices (1 or 2)
    int mbw;      // token blocks of 16 per wave (1 or 2)
    int rb;       // row blocks of 16 per workgroup (1 .. 8)
    int grid;     // workgroups (one per compute unit, a multiple of 8)
    int units;    // weight rows in units of 8
};
RowsPlan plan_gemm_rows(int M, int N, int K, int num_cu);
TileInfo launch_gemm_rows(bool i32_out, const GemmArgs &a, hipStream_t st, bool launch);

// Few-token per-channel product (1 <= M <= 4, M * K <= 64 KiB): the weight
// rows streamed whole against the tokens' codes in LDS; equals the
// per-channel GEMM bit for bit.
void launch_few_pc(const int8_t *xq, const float *xs, const int8_t *w, const float *sw,
                   uint16_t *y, int M, int N, int K, hipStream_t st);

// Few-token W4A8 product (1 <= M <= 4, M * K <= 64 KiB, gs 64 or 128): packed
// int4 rows streamed whole against the tokens' codes in LDS; same results as
// the W4A8 GEMM up to the fp32 summation order over the groups.
void launch_few_w4(const int8_t *xq, const float *xs, const uint8_t *w, const float *sw, int gs,
                   uint16_t *y, int M, int N, int K, hipStream_t st);

// Decode matrix-vector: quantize the token, y[n] = rescale(sum_k q[k] w[n,k]).
void launch_int8_mv(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int N,
                    int K, int8_t *xq_out, float *xs_out, hipStream_t st);

// Decode matrix-vector with per-group weight scales: per-group W8A8 (token
// quantized per group of gs) or W4A8 (packed int4 weights, per-token scale).
// num_cu sizes the rows per workgroup.
void launch_mv_group(bool int4, int gs, const uint16_t *x, const uint8_t *w, const float *sw,
                     uint16_t *y, int N, int K, int num_cu, hipStream_t st);

// Weight-only int8 comparison GEMM: y = fp16(w_scale[n] * sum_k x[m,k] wq[n,k])
// with fp16 activations on the fp16 matrix cores (K % 64 == 0).
void launch_w8a16(const uint16_t *x, const int8_t *w, const float *sw, uint16_t *y, int M, int N,
                  int K, hipStream_t st);
// Weight-only int4 comparison GEMM: y = fp16(sum_k x[m,k] fp16(fl32(code[n,k]
// w_scale[n,g]))) with packed int4 weights [N, K/2] (K % 64 == 0, K % gs == 0).
void launch_w4a16(const uint16_t *x, const uint8_t *w4, const float *sw, int gs, uint16_t *y, int M,
                  int N, int K, hipStream_t st);
// Their decode (M = 1) form: y[n] for one fp16 token x [K] (K <= 16384).
void launch_wo_mv(bool int4, const uint16_t *x, const void *w, const float *sw, int gs, uint16_t *y,
                  int N, int K, hipStream_t st);

}  // namespace w4a8
