// C entry points of libw4a8: argument checks, device check, kernel dispatch.
// The operations and their sources are described in include/w4a8.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/w4a8.h"
#include "kernels.hpp"

using namespace w4a8;

namespace {

thread_local char g_err[512] = "";

w4a8_status_t fail(w4a8_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

w4a8_status_t ok()
{
    g_err[0] = '\0';
    return W4A8_OK;
}

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kMaxKPerChannel = 133144;   // largest K with 127^2 * K < 2^31
constexpr int64_t kMaxKMv = 32768;            // the token's codes are staged in LDS
constexpr int64_t kMaxKWoMv = 16384;          // weight-only decode: the token as fp32 in LDS
constexpr int64_t kMaxKGemm = int64_t(1) << 22; // a 256-row tile of K bytes stays below 2^30
constexpr int64_t kMaxTiles = 0x7fffffff;     // 32 x 128 output tiles
// Few-token per-channel and W4A8 products (the weight rows streamed whole): up
// to 4 tokens, whose codes are staged in LDS
constexpr int64_t kMaxMFew = 4;
constexpr int64_t kMaxFewCodes = 65536;       // M * K bytes

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Per device ordinal: its compute-unit count if it is a gfx950, 0 if it is
// something else, -1 while not yet known.
std::atomic<int> g_dev_cu[64];
struct DevInit {
    DevInit() { for (auto &a : g_dev_cu) a.store(-1); }
} g_dev_init;

// The current device must be a gfx950; *num_cu receives its compute units.
w4a8_status_t check_device(int *num_cu = nullptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return fail(W4A8_ERR_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
    if (dev < 64) {
        const int known = g_dev_cu[dev].load(std::memory_order_relaxed);
        if (known > 0) {
            if (num_cu)
                *num_cu = known;
            return W4A8_OK;
        }
        if (known == 0)
            return fail(W4A8_ERR_DEVICE, "HIP device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(W4A8_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    const bool is950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    const int cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    if (dev < 64)
        g_dev_cu[dev].store(is950 ? cus : 0, std::memory_order_relaxed);
    if (!is950)
        return fail(W4A8_ERR_DEVICE, "HIP device %d is %s, not gfx950", dev, prop.gcnArchName);
    if (num_cu)
        *num_cu = cus;
    return W4A8_OK;
}

w4a8_status_t check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(W4A8_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- argument checks (no HIP calls)

w4a8_status_t check_quant(const char *fn, const void *x, int64_t rows, int64_t K, int32_t gs,
                          const void *q, const float *scale, bool int4)
{
    if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "%s: sizes out of range (rows=%lld K=%lld)", fn,
                    (long long)rows, (long long)K);
    if (K == 0 || K % 8 != 0)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 8", fn, (long long)K);
    if (int4 ? !(gs == 64 || gs == 128) : !(gs == 0 || gs == 64 || gs == 128))
        return fail(W4A8_ERR_SHAPE, "%s: group_size=%d not supported", fn, gs);
    if (gs > 0 && K % gs != 0)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld is not a multiple of group_size=%d", fn,
                    (long long)K, gs);
    if (rows == 0)
        return W4A8_OK;
    if (!x || !q || !scale)
        return fail(W4A8_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale))
        return fail(W4A8_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
    return W4A8_OK;
}

w4a8_status_t check_gemm(const char *fn, const void *xq, const void *w, const void *out,
                         const float *sa, const float *sw, int64_t M, int64_t N, int64_t K,
                         int32_t gs, bool pergroup, bool need_scales)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "%s: sizes out of range (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (K == 0 || K % 64 != 0)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 64", fn,
                    (long long)K);
    if (pergroup) {
        if (!(gs == 64 || gs == 128))
            return fail(W4A8_ERR_SHAPE, "%s: group_size=%d must be 64 or 128", fn, gs);
        if (K % gs != 0)
            return fail(W4A8_ERR_SHAPE, "%s: K=%lld is not a multiple of group_size=%d", fn,
                        (long long)K, gs);
    } else if (K > kMaxKPerChannel) {
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld could overflow the int32 sums (max %lld)", fn,
                    (long long)K, (long long)kMaxKPerChannel);
    }
    if (K > kMaxKGemm)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld exceeds %lld", fn, (long long)K,
                    (long long)kMaxKGemm);
    if (((M + 31) / 32) * ((N + 127) / 128) > kMaxTiles)
        return fail(W4A8_ERR_SHAPE, "%s: output of %lld x %lld is too large", fn, (long long)M,
                    (long long)N);
    if (M == 0 || N == 0)
        return W4A8_OK;
    if (!xq || !w || !out || (need_scales && (!sa || !sw)))
        return fail(W4A8_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned16(xq) || !aligned16(w) || !aligned16(out) ||
        (need_scales && (!aligned4(sa) || !aligned4(sw))))
        return fail(W4A8_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
    return W4A8_OK;
}

w4a8_status_t check_mv(const void *x, const void *w, const float *sw, const void *y, int64_t N,
                       int64_t K, const int8_t *xq_out, const float *xs_out)
{
    if (N < 0 || K < 0 || N > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "int8_mv: sizes out of range");
    if (K == 0 || K % 16 != 0 || K > kMaxKMv)
        return fail(W4A8_ERR_SHAPE, "int8_mv: K=%lld must be a multiple of 16 in (0, %lld]",
                    (long long)K, (long long)kMaxKMv);
    if (!x)
        return fail(W4A8_ERR_INVALID_ARG, "int8_mv: null x");
    if (N > 0 && (!w || !sw || !y))
        return fail(W4A8_ERR_INVALID_ARG, "int8_mv: null pointer");
    if (!aligned16(x) || (N > 0 && (!aligned16(w) || !aligned4(sw) || !aligned4(y))) ||
        (xq_out && !aligned16(xq_out)) || (xs_out && !aligned4(xs_out)))
        return fail(W4A8_ERR_ALIGNMENT, "int8_mv: misaligned tensor");
    return W4A8_OK;
}

w4a8_status_t check_mv_group(const char *fn, const void *x, const void *w, const float *sw,
                             const void *y, int64_t N, int64_t K, int32_t gs)
{
    if (N < 0 || K < 0 || N > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "%s: sizes out of range", fn);
    if (gs != 64 && gs != 128)
        return fail(W4A8_ERR_SHAPE, "%s: group_size %d must be 64 or 128", fn, (int)gs);
    if (K == 0 || K % 64 != 0 || K % gs != 0 || K > kMaxKMv)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a multiple of 64 and of group_size in "
                    "(0, %lld]", fn, (long long)K, (long long)kMaxKMv);
    if (!x || (N > 0 && (!w || !sw || !y)))
        return fail(W4A8_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned16(x) || (N > 0 && (!aligned16(w) || !aligned4(sw) || !aligned4(y))))
        return fail(W4A8_ERR_ALIGNMENT, "%s: misaligned tensor", fn);
    return W4A8_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---- the static scratch of linear_noalloc(): the activations' int8 codes
// and fp32 scales live in this device array instead of a caller workspace.
// Each device the library runs on holds its own copy (placed when the code
// object is loaded there) until the process ends.  Host code never passes
// the array's name to a kernel (on the host it only names the symbol): the
// device address is looked up per device with hipGetSymbolAddress and kept.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<uintptr_t> g_scratch_dev[64];     // per device ordinal; 0 = not looked up yet

// Device address of the current device's copy of `scratch`.
w4a8_status_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64)
        return fail(W4A8_ERR_DEVICE, "no HIP device for the static scratch (%s)",
                    hipGetErrorString(e));
    uintptr_t p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(W4A8_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d failed: %s",
                        dev, hipGetErrorString(e));
        p = reinterpret_cast<uintptr_t>(ptr);
        g_scratch_dev[dev].store(p, std::memory_order_release);
    }
    *out = reinterpret_cast<void *>(p);
    return W4A8_OK;
}

GemmArgs make_args(const int8_t *xq, const float *sa, const void *w, const float *sw, void *out,
                   int64_t M, int64_t N, int64_t K, int gs)
{
    GemmArgs a;
    a.xq = xq; a.sa = sa; a.w = w; a.sw = sw; a.out = out;
    a.M = (int)M; a.N = (int)N; a.K = (int)K; a.gs = gs;
    a.num_cu = 1;
    return a;
}

w4a8_status_t run_gemm(const char *fn, GemmMode mode, const GemmArgs &a, w4a8_stream_t stream)
{
    if (a.M == 0 || a.N == 0)
        return ok();
    GemmArgs la = a;
    w4a8_status_t st = check_device(&la.num_cu);
    if (st != W4A8_OK)
        return st;
    launch_gemm(mode, la, (hipStream_t)stream);
    return check_launch(fn);
}

// The per-channel product on checked arguments: up to four tokens as the
// few-token matrix-vector form (same arithmetic), else the GEMM.
w4a8_status_t run_pc(const char *fn, const int8_t *xq, const float *xs, const int8_t *wq,
                     const float *sw, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                     w4a8_stream_t stream)
{
    if (M >= 1 && M <= kMaxMFew && M * K <= kMaxFewCodes) {
        if (N == 0)
            return ok();
        w4a8_status_t st = check_device();
        if (st != W4A8_OK)
            return st;
        launch_few_pc(xq, xs, wq, sw, y, (int)M, (int)N, (int)K, (hipStream_t)stream);
        return check_launch(fn);
    }
    return run_gemm(fn, GemmMode::PC, make_args(xq, xs, wq, sw, y, M, N, K, 0), stream);
}

// The W4A8 product on checked arguments: up to four tokens as the few-token
// matrix-vector form, else the GEMM.
w4a8_status_t run_w4(const char *fn, const int8_t *xq, const float *xs, const uint8_t *w4,
                     const float *sw, int gs, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                     w4a8_stream_t stream)
{
    if (M >= 1 && M <= kMaxMFew && M * K <= kMaxFewCodes) {
        if (N == 0)
            return ok();
        w4a8_status_t st = check_device();
        if (st != W4A8_OK)
            return st;
        launch_few_w4(xq, xs, w4, sw, gs, y, (int)M, (int)N, (int)K, (hipStream_t)stream);
        return check_launch(fn);
    }
    return run_gemm(fn, GemmMode::W4, make_args(xq, xs, w4, sw, y, M, N, K, gs), stream);
}

w4a8_status_t run_quant(const char *fn, const uint16_t *x, int64_t rows, int64_t K, int gs,
                        float qmax, void *q, float *scale, bool int4, w4a8_stream_t stream)
{
    if (rows == 0)
        return ok();
    w4a8_status_t st = check_device();
    if (st != W4A8_OK)
        return st;
    launch_quantize_rows(x, rows, (int)K, gs, qmax, q, scale, int4, (hipStream_t)stream);
    return check_launch(fn);
}

}  // namespace

namespace {

// linear()'s argument rules (no HIP calls): the mode, then the GEMM's rules,
// whatever M is.  Sets *empty for a call with nothing to do.
w4a8_status_t check_linear(const char *fn, w4a8_mode_t mode, const w4a8_f16 *x, int64_t M,
                           int64_t K, const void *w, const float *w_scale, int32_t group_size,
                           int64_t N, w4a8_f16 *y, bool *empty)
{
    *empty = false;
    if (mode != W4A8_MODE_W8A8_PC && mode != W4A8_MODE_W8A8_PG && mode != W4A8_MODE_W4A8)
        return fail(W4A8_ERR_INVALID_ARG, "%s: unknown mode %d", fn, (int)mode);
    const bool pg = mode != W4A8_MODE_W8A8_PC;
    const int32_t gs = pg ? group_size : 0;
    w4a8_status_t st = check_gemm(fn, x, w, y, w_scale, w_scale, M, N, K, gs, pg, true);
    if (st != W4A8_OK)
        return st;
    if (M == 0 || N == 0) {
        *empty = true;
        return W4A8_OK;
    }
    if (!x || !aligned16(x))
        return fail(x ? W4A8_ERR_ALIGNMENT : W4A8_ERR_INVALID_ARG, "%s: bad x", fn);
    return W4A8_OK;
}

// The layer on checked arguments (check_linear) with the given workspace,
// which may be the static scratch (linear_noalloc).
w4a8_status_t linear_run(const char *fn, w4a8_mode_t mode, const w4a8_f16 *x, int64_t M,
                         int64_t K, const void *w, const float *w_scale, int32_t group_size,
                         int64_t N, w4a8_f16 *y, void *workspace, size_t workspace_bytes,
                         w4a8_stream_t stream)
{
    const int32_t act_gs = (mode == W4A8_MODE_W8A8_PG) ? group_size : 0;
    w4a8_status_t st;
    if (M == 1 && K <= kMaxKMv) {                 // decode: the matrix-vector kernels
        switch (mode) {
        case W4A8_MODE_W8A8_PC:
            return int8_mv(x, static_cast<const int8_t *>(w), w_scale, y, N, K, nullptr, nullptr,
                           stream);
        case W4A8_MODE_W8A8_PG:
            return w8a8_mv_pg(x, static_cast<const int8_t *>(w), w_scale, group_size, y, N, K,
                              stream);
        default:
            return w4a8_mv(x, static_cast<const uint8_t *>(w), w_scale, group_size, y, N, K,
                           stream);
        }
    }
    const size_t need = linear_workspace_size(mode, M, K, group_size);
    if (!workspace || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(W4A8_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) needed, "
                    "got %zu", fn, need, workspace_bytes);
    int8_t *xq = static_cast<int8_t *>(workspace);
    float *xs = reinterpret_cast<float *>(static_cast<char *>(workspace) + align256((size_t)M * K));
    st = quantize_act(x, M, K, act_gs, xq, xs, stream);
    if (st != W4A8_OK)
        return st;
    switch (mode) {
    case W4A8_MODE_W8A8_PC:
        return run_pc(fn, xq, xs, static_cast<const int8_t *>(w), w_scale, y, M, N, K, stream);
    case W4A8_MODE_W8A8_PG:
        return run_gemm(fn, GemmMode::PG,
                        make_args(xq, xs, w, w_scale, y, M, N, K, group_size), stream);
    default:
        return run_w4(fn, xq, xs, static_cast<const uint8_t *>(w), w_scale, group_size, y, M,
                      N, K, stream);
    }
}

}  // namespace

extern "C" {

int w4a8_is_available(void) { return check_device() == W4A8_OK ? 1 : 0; }

const char *w4a8_status_string(w4a8_status_t s)
{
    switch (s) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_INVALID_ARG: return "invalid argument";
    case W4A8_ERR_SHAPE: return "unsupported shape";
    case W4A8_ERR_ALIGNMENT: return "misaligned tensor";
    case W4A8_ERR_DEVICE: return "no gfx950 device";
    case W4A8_ERR_LAUNCH: return "kernel launch failed";
    case W4A8_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

const char *w4a8_last_error(void) { return g_err; }

w4a8_status_t quantize_act(const w4a8_f16 *x, int64_t M, int64_t K, int32_t group_size,
                           int8_t *xq, float *x_scale, w4a8_stream_t stream)
{
    w4a8_status_t st = check_quant("quantize_act", x, M, K, group_size, xq, x_scale, false);
    if (st != W4A8_OK)
        return st;
    return run_quant("quantize_act", x, M, K, group_size, 127.0f, xq, x_scale, false, stream);
}

w4a8_status_t quantize_weight_int8(const w4a8_f16 *w, int64_t N, int64_t K, int32_t group_size,
                                   int8_t *wq, float *w_scale, w4a8_stream_t stream)
{
    w4a8_status_t st = check_quant("quantize_weight_int8", w, N, K, group_size, wq, w_scale, false);
    if (st != W4A8_OK)
        return st;
    return run_quant("quantize_weight_int8", w, N, K, group_size, 127.0f, wq, w_scale, false,
                     stream);
}

w4a8_status_t pack_weight_int4(const w4a8_f16 *w, int64_t N, int64_t K, int32_t group_size,
                               uint8_t *w4, float *w_scale, w4a8_stream_t stream)
{
    w4a8_status_t st = check_quant("pack_weight_int4", w, N, K, group_size, w4, w_scale, true);
    if (st != W4A8_OK)
        return st;
    return run_quant("pack_weight_int4", w, N, K, group_size, 7.0f, w4, w_scale, true, stream);
}

w4a8_status_t w8a8_gemm_pc(const int8_t *xq, const float *x_scale, const int8_t *wq,
                           const float *w_scale, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                           w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w8a8_gemm_pc", xq, wq, y, x_scale, w_scale, M, N, K, 0, false,
                                  true);
    if (st != W4A8_OK)
        return st;
    return run_pc("w8a8_gemm_pc", xq, x_scale, wq, w_scale, y, M, N, K, stream);
}

w4a8_status_t w8a8_gemm_pg(const int8_t *xq, const float *x_scale, const int8_t *wq,
                           const float *w_scale, int32_t group_size, w4a8_f16 *y, int64_t M,
                           int64_t N, int64_t K, w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w8a8_gemm_pg", xq, wq, y, x_scale, w_scale, M, N, K, group_size,
                                  true, true);
    if (st != W4A8_OK)
        return st;
    return run_gemm("w8a8_gemm_pg", GemmMode::PG,
                    make_args(xq, x_scale, wq, w_scale, y, M, N, K, group_size), stream);
}

w4a8_status_t w4a8_gemm(const int8_t *xq, const float *x_scale, const uint8_t *w4,
                        const float *w_scale, int32_t group_size, w4a8_f16 *y, int64_t M,
                        int64_t N, int64_t K, w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w4a8_gemm", xq, w4, y, x_scale, w_scale, M, N, K, group_size,
                                  true, true);
    if (st != W4A8_OK)
        return st;
    return run_w4("w4a8_gemm", xq, x_scale, w4, w_scale, group_size, y, M, N, K, stream);
}

w4a8_status_t int8_mv(const w4a8_f16 *x, const int8_t *wq, const float *w_scale, w4a8_f16 *y,
                      int64_t N, int64_t K, int8_t *xq_out, float *x_scale_out,
                      w4a8_stream_t stream)
{
    w4a8_status_t st = check_mv(x, wq, w_scale, y, N, K, xq_out, x_scale_out);
    if (st != W4A8_OK)
        return st;
    if (N == 0 && !xq_out && !x_scale_out)
        return ok();
    st = check_device();
    if (st != W4A8_OK)
        return st;
    if (N == 0) {
        // nothing to multiply, but the caller asked for the token's codes:
        // the codes come from the activation quantizer (same rule)
        if (!xq_out || !x_scale_out)
            return fail(W4A8_ERR_INVALID_ARG, "int8_mv: N == 0 needs both or neither export");
        launch_quantize_rows(x, 1, (int)K, 0, 127.0f, xq_out, x_scale_out, false,
                             (hipStream_t)stream);
        return check_launch("int8_mv");
    }
    launch_int8_mv(x, wq, w_scale, y, (int)N, (int)K, xq_out, x_scale_out, (hipStream_t)stream);
    return check_launch("int8_mv");
}

w4a8_status_t w8a8_mv_pg(const w4a8_f16 *x, const int8_t *wq, const float *w_scale,
                         int32_t group_size, w4a8_f16 *y, int64_t N, int64_t K,
                         w4a8_stream_t stream)
{
    w4a8_status_t st = check_mv_group("w8a8_mv_pg", x, wq, w_scale, y, N, K, group_size);
    if (st != W4A8_OK)
        return st;
    if (N == 0)
        return ok();
    int cu = 0;
    st = check_device(&cu);
    if (st != W4A8_OK)
        return st;
    launch_mv_group(false, group_size, x, reinterpret_cast<const uint8_t *>(wq), w_scale, y,
                    (int)N, (int)K, cu, (hipStream_t)stream);
    return check_launch("w8a8_mv_pg");
}

w4a8_status_t w4a8_mv(const w4a8_f16 *x, const uint8_t *w4, const float *w_scale,
                      int32_t group_size, w4a8_f16 *y, int64_t N, int64_t K,
                      w4a8_stream_t stream)
{
    w4a8_status_t st = check_mv_group("w4a8_mv", x, w4, w_scale, y, N, K, group_size);
    if (st != W4A8_OK)
        return st;
    if (N == 0)
        return ok();
    int cu = 0;
    st = check_device(&cu);
    if (st != W4A8_OK)
        return st;
    launch_mv_group(true, group_size, x, w4, w_scale, y, (int)N, (int)K, cu, (hipStream_t)stream);
    return check_launch("w4a8_mv");
}

size_t linear_workspace_size(w4a8_mode_t mode, int64_t M, int64_t K, int32_t group_size)
{
    if (M <= 0 || K <= 0)
        return 0;
    if (M == 1 && K <= kMaxKMv)                   // the matrix-vector kernels need none
        return 0;
    int64_t groups = 1;
    if (mode == W4A8_MODE_W8A8_PG && group_size > 0)
        groups = K / group_size;
    return align256((size_t)M * (size_t)K) + align256((size_t)M * (size_t)groups * sizeof(float));
}

w4a8_status_t linear(w4a8_mode_t mode, const w4a8_f16 *x, int64_t M, int64_t K, const void *w,
                     const float *w_scale, int32_t group_size, int64_t N, w4a8_f16 *y,
                     void *workspace, size_t workspace_bytes, w4a8_stream_t stream)
{
    bool empty;
    w4a8_status_t st = check_linear("linear", mode, x, M, K, w, w_scale, group_size, N, y, &empty);
    if (st != W4A8_OK || empty)
        return st == W4A8_OK ? ok() : st;
    return linear_run("linear", mode, x, M, K, w, w_scale, group_size, N, y, workspace,
                      workspace_bytes, stream);
}

w4a8_status_t linear_noalloc(w4a8_mode_t mode, const w4a8_f16 *x, int64_t M, int64_t K,
                             const void *w, const float *w_scale, int32_t group_size, int64_t N,
                             w4a8_f16 *y, w4a8_stream_t stream)
{
    const char *fn = "linear_noalloc";
    bool empty;
    w4a8_status_t st = check_linear(fn, mode, x, M, K, w, w_scale, group_size, N, y, &empty);
    if (st != W4A8_OK || empty)
        return st == W4A8_OK ? ok() : st;
    const size_t need = linear_workspace_size(mode, M, K, group_size);
    if (need > kScratchBytes)
        return fail(W4A8_ERR_WORKSPACE, "%s: M=%lld, K=%lld need %zu bytes of scratch; the "
                    "static array holds %zu (call linear() with a workspace)", fn, (long long)M,
                    (long long)K, need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        st = check_device();
        if (st != W4A8_OK)
            return st;
        st = scratch_address(&ws);
        if (st != W4A8_OK)
            return st;
    }
    return linear_run(fn, mode, x, M, K, w, w_scale, group_size, N, y, ws, kScratchBytes, stream);
}

w4a8_status_t w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int32_t *c, int64_t M, int64_t N,
                            int64_t K, w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w8a8_gemm_i32", xq, wq, c, nullptr, nullptr, M, N, K, 0, false,
                                  false);
    if (st != W4A8_OK)
        return st;
    return run_gemm("w8a8_gemm_i32", GemmMode::I32,
                    make_args(xq, nullptr, wq, nullptr, c, M, N, K, 0), stream);
}

w4a8_status_t w8a8_gemm_pg_partials(const int8_t *xq, const int8_t *wq, int32_t group_size,
                                    int32_t *p, int64_t M, int64_t N, int64_t K,
                                    w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w8a8_gemm_pg_partials", xq, wq, p, nullptr, nullptr, M, N, K,
                                  group_size, true, false);
    if (st != W4A8_OK)
        return st;
    return run_gemm("w8a8_gemm_pg_partials", GemmMode::PG_PARTIALS,
                    make_args(xq, nullptr, wq, nullptr, p, M, N, K, group_size), stream);
}

w4a8_status_t w4a8_gemm_partials(const int8_t *xq, const uint8_t *w4, int32_t group_size,
                                 int32_t *p, int64_t M, int64_t N, int64_t K,
                                 w4a8_stream_t stream)
{
    w4a8_status_t st = check_gemm("w4a8_gemm_partials", xq, w4, p, nullptr, nullptr, M, N, K,
                                  group_size, true, false);
    if (st != W4A8_OK)
        return st;
    return run_gemm("w4a8_gemm_partials", GemmMode::W4_PARTIALS,
                    make_args(xq, nullptr, w4, nullptr, p, M, N, K, group_size), stream);
}

w4a8_status_t w8a16_gemm(const w4a8_f16 *x, const int8_t *wq, const float *w_scale, w4a8_f16 *y,
                         int64_t M, int64_t N, int64_t K, w4a8_stream_t stream)
{
    const char *fn = "w8a16_gemm";
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "%s: sizes out of range (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (K == 0 || K % 64 != 0)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 64", fn,
                    (long long)K);
    if ((M + 127) / 128 > 65535)
        return fail(W4A8_ERR_SHAPE, "%s: M=%lld exceeds 65535 * 128 rows", fn, (long long)M);
    if (M == 0 || N == 0)
        return ok();
    if (!x || !wq || !w_scale || !y)
        return fail(W4A8_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned16(x) || !aligned16(wq) || !aligned16(y) || !aligned4(w_scale))
        return fail(W4A8_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
    w4a8_status_t st = check_device();
    if (st != W4A8_OK)
        return st;
    if (M == 1 && K <= kMaxKWoMv)                     // one token: the matrix-vector form
        launch_wo_mv(false, reinterpret_cast<const uint16_t *>(x), wq, w_scale, 0,
                     reinterpret_cast<uint16_t *>(y), (int)N, (int)K, (hipStream_t)stream);
    else
        launch_w8a16(reinterpret_cast<const uint16_t *>(x), wq, w_scale,
                     reinterpret_cast<uint16_t *>(y), (int)M, (int)N, (int)K, (hipStream_t)stream);
    return check_launch(fn);
}

w4a8_status_t w4a16_gemm(const w4a8_f16 *x, const uint8_t *w4, const float *w_scale,
                         int32_t group_size, w4a8_f16 *y, int64_t M, int64_t N, int64_t K,
                         w4a8_stream_t stream)
{
    const char *fn = "w4a16_gemm";
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(W4A8_ERR_INVALID_ARG, "%s: sizes out of range (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (!(group_size == 64 || group_size == 128))
        return fail(W4A8_ERR_SHAPE, "%s: group_size=%d must be 64 or 128", fn, (int)group_size);
    if (K == 0 || K % 64 != 0 || K % group_size != 0)
        return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 64 and of "
                    "group_size", fn, (long long)K);
    if ((M + 127) / 128 > 65535)
        return fail(W4A8_ERR_SHAPE, "%s: M=%lld exceeds 65535 * 128 rows", fn, (long long)M);
    if (M == 0 || N == 0)
        return ok();
    if (!x || !w4 || !w_scale || !y)
        return fail(W4A8_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned16(x) || !aligned16(w4) || !aligned16(y) || !aligned4(w_scale))
        return fail(W4A8_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
    w4a8_status_t st = check_device();
    if (st != W4A8_OK)
        return st;
    if (M == 1 && K <= kMaxKWoMv)                     // one token: the matrix-vector form
        launch_wo_mv(true, reinterpret_cast<const uint16_t *>(x), w4, w_scale, (int)group_size,
                     reinterpret_cast<uint16_t *>(y), (int)N, (int)K, (hipStream_t)stream);
    else
        launch_w4a16(reinterpret_cast<const uint16_t *>(x), w4, w_scale, (int)group_size,
                     reinterpret_cast<uint16_t *>(y), (int)M, (int)N, (int)K, (hipStream_t)stream);
    return check_launch(fn);
}

w4a8_status_t gemm_tile_config(w4a8_gemm_op_t op, int64_t M, int64_t N, int64_t K,
                               int32_t group_size, int64_t *out)
{
    const char *fn = "gemm_tile_config";
    if (!out)
        return fail(W4A8_ERR_INVALID_ARG, "%s: null out", fn);
    GemmMode mode;
    bool pergroup = true, few = false;
    switch (op) {
    case W4A8_OP_GEMM_PC: mode = GemmMode::PC; pergroup = false; few = true; break;
    case W4A8_OP_GEMM_I32: mode = GemmMode::I32; pergroup = false; break;
    case W4A8_OP_GEMM_PG: mode = GemmMode::PG; break;
    case W4A8_OP_PG_PARTIALS: mode = GemmMode::PG_PARTIALS; break;
    case W4A8_OP_GEMM_W4A8: mode = GemmMode::W4; few = true; break;
    case W4A8_OP_W4A8_PARTIALS: mode = GemmMode::W4_PARTIALS; break;
    default: return fail(W4A8_ERR_INVALID_ARG, "%s: unknown op %d", fn, (int)op);
    }
    // the entry point's own shape rules (pointers are not inspected)
    static const int8_t dummy[16] __attribute__((aligned(16))) = {0};
    const float *fs = reinterpret_cast<const float *>(dummy);
    w4a8_status_t st = check_gemm(fn, dummy, dummy, dummy, fs, fs, M, N, K,
                                  pergroup ? group_size : 0, pergroup, false);
    if (st != W4A8_OK)
        return st;
    for (int i = 0; i < 6; ++i)
        out[i] = 0;
    if (M == 0 || N == 0)
        return ok();
    int num_cu = 0;
    st = check_device(&num_cu);
    if (st != W4A8_OK)
        return st;
    if (few && M >= 1 && M <= kMaxMFew && M * K <= kMaxFewCodes)
        return ok();                              // the few-token matrix-vector form
    GemmArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K,
                           pergroup ? group_size : 0);
    a.num_cu = num_cu;
    const TileInfo t = gemm_info(mode, a);
    out[0] = t.bm;
    out[1] = t.bn;
    out[2] = t.waves;
    out[3] = t.grid;
    out[4] = t.tiles;
    out[5] = t.per_cu;
    return ok();
}

}  // extern "C"
