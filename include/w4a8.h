/*
 * w4a8.h -- C ABI of the MI355X (gfx950) W8A8 / W4A8 int8 linear layer.
 *
 * What is computed (sources are web pages; sections named as printed):
 *  [P1] "Apple Silicon의 AI 한계치는 당신의 생각보다 높습니다" (molayo1419.me),
 *       section "INT8 TensorOps 커널 설계" (INT8 TensorOps kernel design): a
 *       per-input min/max pass yields scale factors, activations are mapped
 *       to INT8 with them in one streaming pass, an INT8 x INT8 GEMM
 *       accumulates in INT32, and the INT32 result is rescaled by the product
 *       of activation and weight scales into an FP16 output.  Section "입도"
 *       (granularity): per-group scales need grouped dequantization during
 *       accumulation.
 *  [P2] "cider: Apple Silicon M5 INT8 TensorOps ... W8A8 SDK"
 *       (discuss.pytorch.kr), section "cider의 양자화 모드와 적용 가능한 영역"
 *       (modes table): W8A8 = symmetric INT8 weights x per-token INT8
 *       activations, in per-channel, per-group gs=128 and gs=64 variants;
 *       W4A8 = INT4 weights packed into uint8, unpacked before the INT8
 *       matmul.  Section "cider의 동작 방식과 자동 경로 선택" (path selection):
 *       a single token goes to an INT8 matrix-vector kernel, longer inputs to
 *       the GEMM.  Section "cider 설치와 사용법" (usage): offline helpers
 *       quantize_weight_int8(W) and pack_weight_int4(W).
 *
 * The quantization rule (one rule for every entry point, activations and
 * weights alike; the pages give no formula, this is the reading taken):
 *     amax = max |x| over the slice (a row, or gs contiguous elements of it)
 *     s    = fl32(amax / qmax)            qmax = 127 (int8) or 7 (int4)
 *     q    = clamp(round_half_away(fl32(x / s)), -qmax, qmax)
 * with IEEE fp32 division; an all-zero slice gets s = 0 and zero codes.
 * Inputs must be finite (not checked).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *    with K contiguous.  Activations, codes, weights and outputs must be
 *    16-byte aligned; fp32 scale vectors 4-byte aligned.  The library
 *    allocates no device memory.  fp16 data is passed as IEEE binary16 bit
 *    patterns (w4a8_f16).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; results are ready when the stream is.
 *    Argument errors return before anything is enqueued; a kernel fault
 *    surfaces at the caller's next synchronisation, as for any HIP launch.
 *  - M == 0 or N == 0 is a valid empty call: nothing is enqueued, W4A8_OK.
 *  - Entry points are re-entrant; no C++ exception crosses the boundary.
 *    w4a8_last_error() gives a thread-local description of the last failure.
 *  - Groups (group_size = gs) are contiguous slices of gs elements along K
 *    starting at k = 0; gs is 64 or 128 and must divide K.
 *  - Packed int4 weights are uint8 [N, K/2]: byte j of row n holds the code of
 *    k = 2j in its low nibble and k = 2j+1 in its high nibble, two's complement.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t w4a8_f16;   /* IEEE binary16 bits */
typedef void *w4a8_stream_t; /* a hipStream_t; NULL is the default stream */

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_INVALID_ARG = 1, /* null pointer for a non-empty tensor, negative size, bad mode */
    W4A8_ERR_SHAPE = 2,       /* K not a multiple of what the kernel needs, bad group size,
                                 K so large that an int32 sum could overflow */
    W4A8_ERR_ALIGNMENT = 3,   /* a tensor base pointer not 16-byte aligned (scales: 4-byte) */
    W4A8_ERR_DEVICE = 4,      /* the current HIP device is not gfx950, or no device */
    W4A8_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch */
    W4A8_ERR_WORKSPACE = 6    /* workspace missing or smaller than linear_workspace_size() */
} w4a8_status_t;

typedef enum {
    W4A8_MODE_W8A8_PC = 0, /* int8 weights, one scale per output channel */
    W4A8_MODE_W8A8_PG = 1, /* int8 weights and activations, scales per group of gs along K */
    W4A8_MODE_W4A8 = 2     /* packed int4 weights with per-group scales, per-token activations */
} w4a8_mode_t;

/* 1 if the current HIP device is a gfx950 (MI355X-class) GPU, else 0
 * ([P2] usage section: the library reports whether its hardware path exists). */
int w4a8_is_available(void);

/* Static English text for a status code. */
const char *w4a8_status_string(w4a8_status_t status);

/* Thread-local detail of the most recent failure on this thread ("" if none). */
const char *w4a8_last_error(void);

/* --------------------------------------------------------------------------
 * Online activation quantization ([P1] kernel design, steps 1-2; [P2] modes
 * table: INT8 per token).  x: fp16 [M, K] -> xq: int8 [M, K] and x_scale:
 * fp32 [M] (group_size 0, one scale per token) or [M, K/group_size]
 * (group_size 64 or 128).  Requires K > 0 and K % 8 == 0.
 * ------------------------------------------------------------------------ */
w4a8_status_t quantize_act(const w4a8_f16 *x, int64_t M, int64_t K, int32_t group_size,
                           int8_t *xq, float *x_scale, w4a8_stream_t stream);

/* Offline int8 weight quantization ([P2] usage: quantize_weight_int8(W) returns
 * int8 codes and scales).  w: fp16 [N, K] -> wq: int8 [N, K], w_scale: fp32
 * [N] (group_size 0, per output channel) or [N, K/group_size].  Same rule and
 * requirements as quantize_act. */
w4a8_status_t quantize_weight_int8(const w4a8_f16 *w, int64_t N, int64_t K, int32_t group_size,
                                   int8_t *wq, float *w_scale, w4a8_stream_t stream);

/* Offline int4 weight quantization and packing ([P2] usage: pack_weight_int4(W)
 * returns packed uint8 weights and scales; modes table: INT4 packed in uint8).
 * w: fp16 [N, K] -> w4: uint8 [N, K/2] (layout above), w_scale: fp32
 * [N, K/group_size]; qmax = 7.  group_size is 64 or 128. */
w4a8_status_t pack_weight_int4(const w4a8_f16 *w, int64_t N, int64_t K, int32_t group_size,
                               uint8_t *w4, float *w_scale, w4a8_stream_t stream);

/* --------------------------------------------------------------------------
 * W8A8 per-channel GEMM ([P1] kernel design, steps 3-4):
 *     y[m, n] = fp16( (sum_k xq[m,k] * wq[n,k]) * x_scale[m] * w_scale[n] )
 * with the sum exact in int32 and the rescale in fp32, rounded to nearest
 * even.  xq int8 [M, K], x_scale fp32 [M], wq int8 [N, K], w_scale fp32 [N],
 * y fp16 [M, N].  Requires K % 64 == 0 and K <= 133144 (so 127^2 K < 2^31).
 * For 1 <= M <= 4 with M*K <= 65536 the product runs as a matrix-vector form
 * that streams whole weight rows (the tokens' codes staged on chip); the
 * arithmetic, and so every output bit, is the same as the GEMM's.
 * ------------------------------------------------------------------------ */
w4a8_status_t w8a8_gemm_pc(const int8_t *xq, const float *x_scale, const int8_t *wq,
                           const float *w_scale, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                           w4a8_stream_t stream);

/* W8A8 per-group GEMM ([P1] granularity section; [P2] per-group gs=128 / 64):
 *     y[m, n] = fp16( sum_g P_g[m,n] * x_scale[m,g] * w_scale[n,g] ),
 *     P_g[m, n] = sum over k in group g of xq[m,k] * wq[n,k]   (exact int32)
 * with the per-group rescale accumulated in fp32.  x_scale fp32 [M, K/gs],
 * w_scale fp32 [N, K/gs]; group_size 64 or 128; K % 64 == 0. */
w4a8_status_t w8a8_gemm_pg(const int8_t *xq, const float *x_scale, const int8_t *wq,
                           const float *w_scale, int32_t group_size, w4a8_f16 *y, int64_t M,
                           int64_t N, int64_t K, w4a8_stream_t stream);

/* W4A8 GEMM ([P2] modes table: INT4 weights unpacked, then the INT8 matmul):
 *     y[m, n] = fp16( x_scale[m] * sum_g P_g[m,n] * w_scale[n,g] ),
 *     P_g[m, n] = sum over k in group g of xq[m,k] * w4code[n,k]
 * xq int8 [M, K] with per-token x_scale fp32 [M]; w4 uint8 [N, K/2] (layout
 * above) with w_scale fp32 [N, K/gs]; group_size 64 or 128; K % 64 == 0.
 * For 1 <= M <= 4 with M*K <= 65536 the product runs as a matrix-vector form
 * that streams whole packed rows (same sums; the fp32 group terms are added in
 * another order, within the same summation bound). */
w4a8_status_t w4a8_gemm(const int8_t *xq, const float *x_scale, const uint8_t *w4,
                        const float *w_scale, int32_t group_size, w4a8_f16 *y, int64_t M,
                        int64_t N, int64_t K, w4a8_stream_t stream);

/* Decode matrix-vector product ([P2] path selection: a single token takes
 * the INT8 MV kernel; file list: per-channel W8A8 MV).  Quantizes the one
 * token x fp16 [K] per the rule above and returns
 *     y[n] = fp16( (sum_k q[k] * wq[n,k]) * s * w_scale[n] ),
 * bit-identical to quantize_act + w8a8_gemm_pc at M = 1.  wq int8 [N, K],
 * w_scale fp32 [N], y fp16 [N].  xq_out (int8 [K]) and x_scale_out (fp32 [1])
 * may be NULL; if given they receive the token's codes and scale.
 * Requires K % 16 == 0 and 0 < K <= 32768. */
w4a8_status_t int8_mv(const w4a8_f16 *x, const int8_t *wq, const float *w_scale, w4a8_f16 *y,
                      int64_t N, int64_t K, int8_t *xq_out, float *x_scale_out,
                      w4a8_stream_t stream);

/* Decode matrix-vector products with per-group weight scales (the decode
 * side of the per-group and W4A8 modes; [P2] file list: a per-group W8A8 MV
 * next to the per-channel one).  Same results as quantize_act + the mode's
 * GEMM at M = 1, up to the fp32 summation order (within the per-group
 * tolerance of the GEMMs):
 *   w8a8_mv_pg: the token is quantized per group of group_size (x_scale[g]);
 *       y[n] = fp16( sum_g P_g[n] * x_scale[g] * w_scale[n,g] ),
 *       wq int8 [N, K], w_scale fp32 [N, K/gs].
 *   w4a8_mv: the token is quantized per token (scale s);
 *       y[n] = fp16( s * sum_g P_g[n] * w_scale[n,g] ),
 *       w4 uint8 [N, K/2] (layout above), w_scale fp32 [N, K/gs].
 * P_g[n] = sum over k in group g of q[k] * w[n,k] (exact int32).  x fp16
 * [K], y fp16 [N].  group_size 64 or 128; K a multiple of 64 and of
 * group_size, 0 < K <= 32768.  N == 0 returns W4A8_OK with no launch. */
w4a8_status_t w8a8_mv_pg(const w4a8_f16 *x, const int8_t *wq, const float *w_scale,
                         int32_t group_size, w4a8_f16 *y, int64_t N, int64_t K,
                         w4a8_stream_t stream);
w4a8_status_t w4a8_mv(const w4a8_f16 *x, const uint8_t *w4, const float *w_scale,
                      int32_t group_size, w4a8_f16 *y, int64_t N, int64_t K,
                      w4a8_stream_t stream);

/* Bytes of device workspace linear() needs for these sizes (int8 codes and
 * fp32 scales of the activations, each 256-byte aligned).  0 when M == 0, and
 * for M == 1 with K <= 32768 (the matrix-vector paths need none). */
size_t linear_workspace_size(w4a8_mode_t mode, int64_t M, int64_t K, int32_t group_size);

/* The whole layer with path selection ([P2] path selection): M == 1 runs the
 * mode's matrix-vector kernel (int8_mv, w8a8_mv_pg or w4a8_mv; K <= 32768);
 * otherwise quantize_act then the mode's product (w8a8_gemm_pc, w8a8_gemm_pg or
 * w4a8_gemm, which themselves stream whole weight rows for up to four tokens).
 * What linear accepts does not depend on M: the GEMM's rules.
 * x fp16 [M, K]; w is int8 [N, K] (PC, PG) or packed uint8 [N, K/2] (W4A8);
 * w_scale as the mode's GEMM takes it; group_size is ignored in PC mode.
 * workspace: device buffer of at least linear_workspace_size() bytes, 256-byte
 * aligned (may be NULL when that size is 0). */
w4a8_status_t linear(w4a8_mode_t mode, const w4a8_f16 *x, int64_t M, int64_t K, const void *w,
                     const float *w_scale, int32_t group_size, int64_t N, w4a8_f16 *y,
                     void *workspace, size_t workspace_bytes, w4a8_stream_t stream);

/* linear() for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same argument rules, kernels and results as linear(), without a workspace
 * argument.  The activations' int8 codes and fp32 scales are kept in a
 * static device array of 64 MiB (2^26 bytes) that the library holds on each
 * GPU it runs on until the process ends; its device address is looked up
 * once per GPU.  A call whose linear_workspace_size() exceeds 64 MiB returns
 * W4A8_ERR_WORKSPACE before anything is launched (use linear() with a
 * workspace instead).  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array and overwrites it: calls that overlap on one GPU
 * (different streams or threads) race, so the caller must order them, e.g.
 * on one stream.  Nothing in the array has to start at zero -- each call
 * writes the codes and scales it then reads. */
w4a8_status_t linear_noalloc(w4a8_mode_t mode, const w4a8_f16 *x, int64_t M, int64_t K,
                             const void *w, const float *w_scale, int32_t group_size, int64_t N,
                             w4a8_f16 *y, w4a8_stream_t stream);

/* --------------------------------------------------------------------------
 * Raw-accumulator exports, for checking the int32 sums bit for bit.  Same
 * main loops as the GEMMs above with the rescale replaced by a store.
 * ------------------------------------------------------------------------ */

/* c int32 [M, N] = xq [M, K] . wq [N, K]^T.  Requirements as w8a8_gemm_pc. */
w4a8_status_t w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int32_t *c, int64_t M, int64_t N,
                            int64_t K, w4a8_stream_t stream);

/* p int32 [K/gs, M, N]: per-group partial sums of the per-group GEMM. */
w4a8_status_t w8a8_gemm_pg_partials(const int8_t *xq, const int8_t *wq, int32_t group_size,
                                    int32_t *p, int64_t M, int64_t N, int64_t K,
                                    w4a8_stream_t stream);

/* p int32 [K/gs, M, N]: per-group partial sums of the W4A8 GEMM (int4 codes
 * unpacked from w4 uint8 [N, K/2]). */
w4a8_status_t w4a8_gemm_partials(const int8_t *xq, const uint8_t *w4, int32_t group_size,
                                 int32_t *p, int64_t M, int64_t N, int64_t K,
                                 w4a8_stream_t stream);

/* --------------------------------------------------------------------------
 * Which kernel configuration a GEMM entry point runs (introspection: tests
 * assert the configuration their shapes exercise; callers can log it).
 * ------------------------------------------------------------------------ */
typedef enum {
    W4A8_OP_GEMM_PC = 0,       /* w8a8_gemm_pc */
    W4A8_OP_GEMM_PG = 1,       /* w8a8_gemm_pg */
    W4A8_OP_GEMM_W4A8 = 2,     /* w4a8_gemm */
    W4A8_OP_GEMM_I32 = 3,      /* w8a8_gemm_i32 */
    W4A8_OP_PG_PARTIALS = 4,   /* w8a8_gemm_pg_partials */
    W4A8_OP_W4A8_PARTIALS = 5  /* w4a8_gemm_partials */
} w4a8_gemm_op_t;

/* For a call of `op` with these sizes on the current device, writes
 *   out[0] = rows of the output tile a workgroup computes (0: the call runs
 *            the few-token matrix-vector form instead of the tiled GEMM; the
 *            row-range forms for a few to a few hundred tokens: the tokens a
 *            workgroup takes, padded),
 *   out[1] = columns of that tile (row-range forms: the weight rows a
 *            workgroup takes in one pass, padded to 16),
 *   out[2] = wavefronts per workgroup,
 *   out[3] = workgroups launched (the grid is persistent: at most as many as
 *            the device holds at once; each walks its share of the tiles),
 *   out[4] = tiles of the M x N output,
 *   out[5] = workgroups the device holds at once per compute unit.
 * Argument rules and errors are those of the entry point itself; nothing is
 * launched.  out is a host array of 6 int64_t. */
w4a8_status_t gemm_tile_config(w4a8_gemm_op_t op, int64_t M, int64_t N, int64_t K,
                               int32_t group_size, int64_t *out);

/* --------------------------------------------------------------------------
 * Weight-only int8 comparison GEMM (W8A16): the baseline of the "cider"
 * post's latency table (section on its performance results, which sets
 * per-channel W8A8 against MLX's weight-only int8 product at N=10240,
 * K=2560).  Activations stay fp16; the int8 codes are used as fp16 values
 * (exact) on the fp16 matrix cores with fp32 accumulation:
 *     y[m, n] = fp16( w_scale[n] * sum_k x[m,k] * wq[n,k] ).
 * x fp16 [M, K], wq int8 [N, K] and w_scale fp32 [N] as produced by
 * quantize_weight_int8 with group_size 0, y fp16 [M, N].  Requires
 * K % 64 == 0 and M <= 65535 * 128; x, wq and y 16-byte aligned.  M == 0 or
 * N == 0 returns W4A8_OK with no launch.  M == 1 with K <= 16384 runs a
 * matrix-vector kernel (the table's one-token row), larger M the GEMM.  Not
 * part of the W8A8 hot path: it exists to measure the W8A8 speed-up the
 * pages report, on this GPU.
 * ------------------------------------------------------------------------ */
w4a8_status_t w8a16_gemm(const w4a8_f16 *x, const int8_t *wq, const float *w_scale,
                         w4a8_f16 *y, int64_t M, int64_t N, int64_t K, w4a8_stream_t stream);

/* Weight-only int4 comparison GEMM (W4A16), the latency table's other
 * baseline (MLX's weight-only int4 product).  Each weight is dequantized to
 * fp16 with its group's scale before the fp16 product:
 *     y[m, n] = fp16( sum_k x[m,k] * fp16(fl32(code[n,k] * w_scale[n,g])) ),
 * fp32 accumulation.  x fp16 [M, K]; w4 uint8 [N, K/2] and w_scale fp32
 * [N, K/group_size] as produced by pack_weight_int4; group_size 64 or 128;
 * K % 64 == 0 and K % group_size == 0; M <= 65535 * 128.  Same conventions
 * as w8a16_gemm, including the matrix-vector form at M == 1. */
w4a8_status_t w4a16_gemm(const w4a8_f16 *x, const uint8_t *w4, const float *w_scale,
                         int32_t group_size, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                         w4a8_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
