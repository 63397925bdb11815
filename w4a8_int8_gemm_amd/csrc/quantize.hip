// Online activation quantization and offline weight quantization kernels.
//
// Steps 1-2 of the kernel pipeline in the Apple-silicon essay ("Apple Silicon의
// AI 한계치는 당신의 생각보다 높습니다", section "INT8 TensorOps 커널 설계"): a
// min/max reduction gives each slice its scale, then one streaming pass maps
// the fp16 values to INT8.  Per-token slices are whole rows; per-group slices
// are gs = 64 or 128 contiguous elements ("cider" post, modes section).
//
// Both passes are fused: one wavefront owns a row, loads it once with 16-byte
// coalesced loads (lane l takes 16-byte chunks l, l+64, ...), reduces |x| with
// a lane butterfly, and writes 8-byte packed codes.  The kernel is bound by
// HBM bandwidth: per element it reads 2 bytes and writes 1.
#include "kernels.hpp"

namespace w4a8 {

namespace {

// Per-token, row held in registers: CPL 16-byte chunks per lane (K <= 512*CPL;
// FULL: K == 512*CPL, every lane's chunks exist and need no bounds checks).
template <int CPL, bool FULL>
__global__ __launch_bounds__(256) void quant_token_kernel(const uint16_t *__restrict__ x,
                                                          int8_t *__restrict__ q,
                                                          float *__restrict__ scale,
                                                          int64_t rows, int K, float qmax)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nch = K >> 3;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + row * (int64_t)K);
    uint4 v[CPL];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if constexpr (FULL)
            v[j] = load_nt(xr + c);
        else
            v[j] = (c < nch) ? load_nt(xr + c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
        m = max(m, absmax_bits8(v[j]));
    m = group_max_u32<64>(m);
    const float amax = h2f((uint16_t)m);
    const float s = quant_scale(amax, qmax);
    const float r = 1.0f / s;
    if (lane == 0)
        scale[row] = s;
    uint2 *qr = reinterpret_cast<uint2 *>(q + row * (int64_t)K);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (FULL || c < nch)
            qr[c] = quant_chunk8(v[j], s, r, qmax);
    }
}

// Per-token, any K: a reduction pass then a quantization pass (the second
// read of the row is served from cache).
__global__ __launch_bounds__(256) void quant_token_loop_kernel(const uint16_t *__restrict__ x,
                                                               int8_t *__restrict__ q,
                                                               float *__restrict__ scale,
                                                               int64_t rows, int K, float qmax)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nch = K >> 3;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + row * (int64_t)K);
    uint32_t m = 0;
    for (int c = lane; c < nch; c += 64)
        m = max(m, absmax_bits8(xr[c]));
    m = group_max_u32<64>(m);
    const float s = quant_scale(h2f((uint16_t)m), qmax);
    const float r = 1.0f / s;
    if (lane == 0)
        scale[row] = s;
    uint2 *qr = reinterpret_cast<uint2 *>(q + row * (int64_t)K);
    for (int c = lane; c < nch; c += 64)
        qr[c] = quant_chunk8(xr[c], s, r, qmax);
}

// Per-group: GCH = gs/8 consecutive lanes own one group, so every 64-lane
// step covers whole groups and the row is processed in a single pass.
// INT4 packs two codes per byte (low nibble = even k) instead of one.
template <int GCH, bool INT4>
__global__ __launch_bounds__(256) void quant_group_kernel(const uint16_t *__restrict__ x,
                                                          uint8_t *__restrict__ q,
                                                          float *__restrict__ scale,
                                                          int64_t rows, int K, float qmax)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int nch = K >> 3;
    const int G = nch / GCH;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + row * (int64_t)K);
    for (int base = 0; base < nch; base += 64) {
        const int c = base + lane;
        const bool valid = c < nch;                  // whole groups are valid or not
        const uint4 v = valid ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t m = group_max_u32<GCH>(absmax_bits8(v));
        const float s = quant_scale(h2f((uint16_t)m), qmax);
        const float r = 1.0f / s;
        if (!valid)
            continue;
        if ((lane % GCH) == 0)
            scale[row * (int64_t)G + c / GCH] = s;
        const uint2 codes = quant_chunk8(v, s, r, qmax);
        if constexpr (INT4) {
            // bytes of `codes` are k = 0..7 of the chunk; pack pairs into nibbles
            const uint32_t lo = codes.x, hi = codes.y;
            const uint32_t p = ((lo & 0xfu) | ((lo >> 4) & 0xf0u)) |
                               (((lo >> 16) & 0xfu) << 8) | (((lo >> 24) & 0xfu) << 12) |
                               ((hi & 0xfu) << 16) | (((hi >> 8) & 0xfu) << 20) |
                               (((hi >> 16) & 0xfu) << 24) | (((hi >> 24) & 0xfu) << 28);
            reinterpret_cast<uint32_t *>(q + row * (int64_t)(K / 2))[c] = p;
        } else {
            reinterpret_cast<uint2 *>(q + row * (int64_t)K)[c] = codes;
        }
    }
}

template <int CPL>
void launch_token(const uint16_t *x, int8_t *q, float *s, int64_t rows, int K, float qmax,
                  hipStream_t st)
{
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (K == 512 * CPL)
        hipLaunchKernelGGL((quant_token_kernel<CPL, true>), dim3(blocks), dim3(256), 0, st, x, q,
                           s, rows, K, qmax);
    else
        hipLaunchKernelGGL((quant_token_kernel<CPL, false>), dim3(blocks), dim3(256), 0, st, x, q,
                           s, rows, K, qmax);
}

}  // namespace

void launch_quantize_rows(const uint16_t *x, int64_t rows, int K, int gs, float qmax, void *q,
                          float *scale, bool int4, hipStream_t st)
{
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    if (gs == 0) {
        int8_t *q8 = static_cast<int8_t *>(q);
        const int cpl = (K + 511) / 512;
        switch (cpl) {
        case 1: launch_token<1>(x, q8, scale, rows, K, qmax, st); return;
        case 2: launch_token<2>(x, q8, scale, rows, K, qmax, st); return;
        case 3: launch_token<3>(x, q8, scale, rows, K, qmax, st); return;
        case 4: launch_token<4>(x, q8, scale, rows, K, qmax, st); return;
        case 5: launch_token<5>(x, q8, scale, rows, K, qmax, st); return;
        case 6: launch_token<6>(x, q8, scale, rows, K, qmax, st); return;
        case 7: case 8: launch_token<8>(x, q8, scale, rows, K, qmax, st); return;
        case 9: case 10: case 11: case 12: launch_token<12>(x, q8, scale, rows, K, qmax, st); return;
        case 13: case 14: case 15: case 16: launch_token<16>(x, q8, scale, rows, K, qmax, st); return;
        case 17: case 18: case 19: case 20: case 21: case 22: case 23: case 24:
            launch_token<24>(x, q8, scale, rows, K, qmax, st); return;
        case 25: case 26: case 27: case 28: case 29: case 30: case 31: case 32:
            launch_token<32>(x, q8, scale, rows, K, qmax, st); return;
        default:
            hipLaunchKernelGGL(quant_token_loop_kernel, dim3(blocks), dim3(256), 0, st, x, q8, scale,
                               rows, K, qmax);
            return;
        }
    }
    uint8_t *qb = static_cast<uint8_t *>(q);
    if (gs == 64) {
        if (int4)
            hipLaunchKernelGGL((quant_group_kernel<8, true>), dim3(blocks), dim3(256), 0, st, x, qb,
                               scale, rows, K, qmax);
        else
            hipLaunchKernelGGL((quant_group_kernel<8, false>), dim3(blocks), dim3(256), 0, st, x, qb,
                               scale, rows, K, qmax);
    } else {
        if (int4)
            hipLaunchKernelGGL((quant_group_kernel<16, true>), dim3(blocks), dim3(256), 0, st, x,
                               qb, scale, rows, K, qmax);
        else
            hipLaunchKernelGGL((quant_group_kernel<16, false>), dim3(blocks), dim3(256), 0, st, x,
                               qb, scale, rows, K, qmax);
    }
}

}  // namespace w4a8
