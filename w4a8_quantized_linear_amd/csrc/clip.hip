// Weight quantization with percentile clipping (Cider README, ossradar.top
// repo page, "LLM Quantization: Precision vs. Speed" note: besides plain
// min-max the scale can come from a percentile, clip_percentile=99.9).
//
// A row's (or group's) range -- the value that takes the absmax's place in
// s = range / 127 (or / 7) -- is the p-th percentile of its |w|: linear
// interpolation between the order statistics of ranks r0 and r1 = r0 + 1
// around the fractional rank (n - 1) * p / 100 with weight g, the default
// method of numpy.percentile (ranks and weight come from the host; the
// interpolation follows numpy's fp64 steps, a + (b - a) g for g < 0.5 and
// b - (b - a)(1 - g) otherwise), rounded to fp32.  Values beyond the range
// saturate at the end codes.
//
// One wavefront per row.  fp16 magnitudes are 15-bit keys whose integer
// order is their value order, so the two order statistics are found exactly
// by two histogram passes over the row in LDS:
//   level 1: 256 bins of key >> 7; a prefix sum across the wavefront finds
//            the bins holding ranks r0 and r1;
//   level 2: 128 bins of key & 127, counted only for keys in those bins.
// A third pass quantizes the row with the resulting scale (the same
// correctly rounded quotient and rint as the plain quantizer).
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront each

__device__ __forceinline__ int wave_inclusive_sum(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o)
            v += t;
    }
    return v;
}

// Bin holding rank r (0-based) of a histogram whose bins are dealt B per
// lane (bins B*lane .. B*lane + B-1), and the count of keys in lower bins.
// Wavefront-uniform results; r must be below the histogram's total.
template <int B>
__device__ __forceinline__ void locate(const int *hist, int r, int lane, int &bin, int &below)
{
    int c[B], sum = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) {
        c[i] = hist[B * lane + i];
        sum += c[i];
    }
    const int incl = wave_inclusive_sum(sum, lane);
    const bool mine = incl - sum <= r && r < incl;
    int b = 0, base = incl - sum, at = 0;
    if (mine) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            if (r < base + c[i]) {
                b = B * lane + i;
                at = base;
                break;
            }
            base += c[i];
        }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    bin = __shfl(b, src, 64);
    below = __shfl(at, src, 64);
}

// numpy's linear interpolation, operation by operation (no contraction).
__device__ __attribute__((noinline)) double lerp_percentile(double a, double b, double g)
{
#pragma clang fp contract(off)
    const double d = b - a;
    return g >= 0.5 ? b - d * (1.0 - g) : a + d * g;
}

template <int BITS, int DT>
__global__ __launch_bounds__(64 * kRowsPerBlock) void clip_quantize_kernel(
    const uint16_t *__restrict__ w, int64_t rows, int len, int r0, int r1, double g,
    uint8_t *__restrict__ out, float *__restrict__ scale)
{
    __shared__ int hist[kRowsPerBlock][512];  // per wavefront: level 1 [256], level 2 [2][128]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
    const bool active = row < rows;  // wavefront-uniform; every wavefront meets the barriers
    int *h1 = hist[wave], *h2 = hist[wave] + 256;
    for (int i = lane; i < 512; i += 64)
        h1[i] = 0;
    __syncthreads();

    const uint16_t *xr = w + (active ? row : 0) * (int64_t)len;
    const int nch = len >> 3;
    if (active) {
        for (int c = lane; c < nch; c += 64) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xr + (int64_t)c * 8);
            const uint32_t k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                atomicAdd(&h1[(k[j] & 0x7FFFu) >> 7], 1);
                atomicAdd(&h1[(k[j] >> 23) & 0xFFu], 1);
            }
        }
    }
    __syncthreads();
    int b0 = 0, below0 = 0, b1 = 0, below1 = 0;
    if (active) {
        locate<4>(h1, r0, lane, b0, below0);
        locate<4>(h1, r1, lane, b1, below1);
        for (int c = lane; c < nch; c += 64) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xr + (int64_t)c * 8);
            const uint32_t k[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t key = (k[j / 2] >> (16 * (j % 2))) & 0x7FFFu;
                const int hi = (int)(key >> 7);
                if (hi == b0)
                    atomicAdd(&h2[key & 127u], 1);
                else if (hi == b1)
                    atomicAdd(&h2[128 + (key & 127u)], 1);
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    int l0, l1, unused;
    locate<2>(h2, r0 - below0, lane, l0, unused);
    if (b1 == b0)
        locate<2>(h2, r1 - below0, lane, l1, unused);
    else
        locate<2>(h2 + 128, r1 - below1, lane, l1, unused);
    const double a = (double)widen_bits<DT>((uint32_t)((b0 << 7) | l0));
    const double b = (double)widen_bits<DT>((uint32_t)((b1 << 7) | l1));
    const float range = (float)lerp_percentile(a, b, g);
    const float s = range / quant_divisor<BITS>();
    if (lane == 0)
        scale[row] = s;
    for (int c = lane; c < nch; c += 64) {
        const uint2 q = quantize_chunk_div<BITS, DT>(*reinterpret_cast<const uint4 *>(xr + (int64_t)c * 8), s);
        if constexpr (BITS == 8)
            *reinterpret_cast<uint2 *>(out + row * len + (int64_t)c * 8) = q;
        else
            *reinterpret_cast<uint32_t *>(out + row * (len / 2) + (int64_t)c * 4) = q.x;
    }
}

template <int BITS, int DT>
hipError_t launch_clip(const uint16_t *w, int64_t rows, int64_t len, int64_t r0, int64_t r1,
                       double g, void *out, float *scale, hipStream_t stream)
{
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kRowsPerBlock);
    hipLaunchKernelGGL((clip_quantize_kernel<BITS, DT>), grid, block, 0, stream, w, rows, (int)len,
                       (int)r0, (int)r1, g, static_cast<uint8_t *>(out), scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_clip_quantize_rows(const uint16_t *w, int dtype, int64_t rows, int64_t len,
                                     int64_t r0, int64_t r1, double g, int bits, void *out,
                                     float *scale, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    if (dtype == DT_BF16)
        return bits == 8 ? launch_clip<8, DT_BF16>(w, rows, len, r0, r1, g, out, scale, stream)
                         : launch_clip<4, DT_BF16>(w, rows, len, r0, r1, g, out, scale, stream);
    return bits == 8 ? launch_clip<8, DT_F16>(w, rows, len, r0, r1, g, out, scale, stream)
                     : launch_clip<4, DT_F16>(w, rows, len, r0, r1, g, out, scale, stream);
}

}  // namespace cider
