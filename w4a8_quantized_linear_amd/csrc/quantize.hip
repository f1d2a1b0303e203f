// Row-wise symmetric quantization kernels: per-token activations (Cider
// README, ossradar.top repo page, "Metal Kernel Pipeline": FP16 activations
// -> INT8 + per-token scales) and the offline weight quantizers ("Low-Level
// API": quantize_weight_int8, pack_weight_int4; "W8A8 Quantization
// Granularity": per channel or per group of 64 / 128).
//
// A "team" of TS lanes owns one row: it loads the row once in 16-byte
// chunks (8 fp16 per lane per chunk, adjacent lanes adjacent in memory),
// keeps it in registers, reduces the absmax with cross-lane shuffles, then
// writes the codes (8 bytes or 4 packed bytes per chunk, again contiguous
// across lanes) and the scale.  Short rows (weight groups of 64 / 128) use
// teams of 8 / 16 lanes so a wavefront still covers 512 bytes per load.
// Rows longer than the register budget take a two-pass kernel that re-reads
// the row from cache.
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

template <int TS, int NCH, int BITS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *__restrict__ x,
                                                            int64_t rows, int64_t len, int64_t ld,
                                                            uint8_t *__restrict__ out,
                                                            float *__restrict__ scale)
{
    constexpr int TEAMS = 256 / TS;
    const int lane = threadIdx.x % TS;
    const int64_t row = (int64_t)blockIdx.x * TEAMS + threadIdx.x / TS;
    if (row >= rows)
        return;  // a team never straddles a wavefront, so whole teams leave together
    const uint16_t *xr = x + row * ld;
    const int nch = (int)(len >> 3);
    uint4 v[NCH];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = i * TS + lane;
        v[i] = c < nch ? *reinterpret_cast<const uint4 *>(xr + (int64_t)c * 8) : uint4{0, 0, 0, 0};
        const uint32_t m = chunk_absmax_bits(v[i]);
        amax = m > amax ? m : amax;
    }
#pragma unroll
    for (int o = TS / 2; o > 0; o >>= 1) {
        const uint32_t other = (uint32_t)__shfl_xor((int)amax, o, TS);
        amax = other > amax ? other : amax;
    }
    const float s = half_bits_to_float(amax) / quant_divisor<BITS>();
    if (lane == 0)
        scale[row] = s;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = i * TS + lane;
        if (c < nch) {
            const uint2 q = quantize_chunk_div<BITS>(v[i], s);
            if constexpr (BITS == 8)
                *reinterpret_cast<uint2 *>(out + row * len + (int64_t)c * 8) = q;
            else
                *reinterpret_cast<uint32_t *>(out + row * (len / 2) + (int64_t)c * 4) = q.x;
        }
    }
}

// One workgroup per row, any length: absmax pass, then a quantize pass that
// reads the row again.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_long_rows_kernel(const uint16_t *__restrict__ x,
                                                                 int64_t len, int64_t ld,
                                                                 uint8_t *__restrict__ out,
                                                                 float *__restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * ld;
    const int64_t nch = len >> 3;
    uint32_t amax = 0;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint32_t m = chunk_absmax_bits(*reinterpret_cast<const uint4 *>(xr + c * 8));
        amax = m > amax ? m : amax;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t other = (uint32_t)__shfl_xor((int)amax, o, 64);
        amax = other > amax ? other : amax;
    }
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
        amax = red[w] > amax ? red[w] : amax;
    const float s = half_bits_to_float(amax) / quant_divisor<BITS>();
    const float rs = 1.0f / s;
    if (threadIdx.x == 0)
        scale[row] = s;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint2 q = quantize_chunk<BITS>(*reinterpret_cast<const uint4 *>(xr + c * 8), s, rs);
        if constexpr (BITS == 8)
            *reinterpret_cast<uint2 *>(out + row * len + c * 8) = q;
        else
            *reinterpret_cast<uint32_t *>(out + row * (len / 2) + c * 4) = q.x;
    }
}

template <int TS, int NCH, int BITS>
hipError_t launch_team(const uint16_t *x, int64_t rows, int64_t len, int64_t ld, void *out,
                       float *scale, hipStream_t stream)
{
    constexpr int TEAMS = 256 / TS;
    const int64_t blocks = (rows + TEAMS - 1) / TEAMS;
    hipLaunchKernelGGL((quantize_rows_kernel<TS, NCH, BITS>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, x, rows, len, ld, static_cast<uint8_t *>(out), scale);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const uint16_t *x, int64_t rows, int64_t len, int64_t ld, void *out,
                       float *scale, hipStream_t stream)
{
    const int64_t nch = len / 8;
    if (nch <= 8)
        return launch_team<8, 1, BITS>(x, rows, len, ld, out, scale, stream);
    if (nch <= 16)
        return launch_team<16, 1, BITS>(x, rows, len, ld, out, scale, stream);
    if (nch <= 32)
        return launch_team<32, 1, BITS>(x, rows, len, ld, out, scale, stream);
    const int64_t per_lane = (nch + 63) / 64;
#define CIDER_TEAM64(n)                                                                   \
    if (per_lane <= n)                                                                    \
        return launch_team<64, n, BITS>(x, rows, len, ld, out, scale, stream);
    CIDER_TEAM64(1)
    CIDER_TEAM64(2)
    CIDER_TEAM64(3)
    CIDER_TEAM64(4)
    CIDER_TEAM64(5)
    CIDER_TEAM64(6)
    CIDER_TEAM64(8)
    CIDER_TEAM64(10)
    CIDER_TEAM64(12)
    CIDER_TEAM64(16)
    CIDER_TEAM64(20)
    CIDER_TEAM64(24)
#undef CIDER_TEAM64
    hipLaunchKernelGGL((quantize_long_rows_kernel<BITS>), dim3((unsigned)rows), dim3(256), 0,
                       stream, x, len, ld, static_cast<uint8_t *>(out), scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t len, int64_t ld,
                                int bits, void *out, float *scale, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    return bits == 8 ? launch_bits<8>(x, rows, len, ld, out, scale, stream)
                     : launch_bits<4>(x, rows, len, ld, out, scale, stream);
}

}  // namespace cider
