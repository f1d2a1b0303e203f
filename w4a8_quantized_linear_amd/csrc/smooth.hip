// SmoothQuant's weight side (Cider README, ossradar.top repo page: SmoothQuant
// named among the preprocessing methods that make a model quantization-
// friendly): the activations of input channel k are divided by a smoothing
// factor s_k inside the activation quantizer, and the weights absorb it
// offline, W' = W diag(s).  This kernel is that fold:
//   w'[n, k] = w[n, k] * s_k, the exact product rounded once, to nearest
//   even, to the weight's own type (fp16 or bf16).
// The product of a 16-bit element (at most 11 significant bits) and an fp32
// factor (24 bits) is exact in fp64.  It is rounded to fp32 toward zero with
// the lowest bit set when inexact ("round to odd"), then to the 16-bit type
// to nearest even: with at least two more bits in the intermediate than in
// the target, that double rounding equals one correct rounding.
//
// Elementwise and HBM-bound: each thread takes 8 consecutive elements (a
// 16-byte load and store), grid-stride over the matrix.
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

template <int DT>
__device__ __forceinline__ uint32_t fold_one(uint32_t h, float s)
{
    const double p = (double)widen_bits<DT>(h) * (double)s;  // exact
    float f = __double2float_rz(p);
    if ((double)f != p)
        f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) | 1u);  // round to odd
    if constexpr (DT == DT_BF16)
        return out_bits<OUT_BF16>(f);
    else
        return out_bits<OUT_F16>(f);
}

template <int DT>
__global__ __launch_bounds__(256) void smooth_fold_kernel(const uint16_t *__restrict__ w, int64_t N,
                                                          int64_t K, const float *__restrict__ sm,
                                                          uint16_t *__restrict__ out)
{
    const int64_t chunks = N * K / 8;  // K % 8 == 0: a chunk never crosses a row
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * 256) {
        const uint4 v = *reinterpret_cast<const uint4 *>(w + c * 8);
        const int64_t k = (c * 8) % K;
        const float4 a = *reinterpret_cast<const float4 *>(sm + k);
        const float4 b = *reinterpret_cast<const float4 *>(sm + k + 4);
        uint4 o;
        o.x = fold_one<DT>(v.x, a.x) | (fold_one<DT>(v.x >> 16, a.y) << 16);
        o.y = fold_one<DT>(v.y, a.z) | (fold_one<DT>(v.y >> 16, a.w) << 16);
        o.z = fold_one<DT>(v.z, b.x) | (fold_one<DT>(v.z >> 16, b.y) << 16);
        o.w = fold_one<DT>(v.w, b.z) | (fold_one<DT>(v.w >> 16, b.w) << 16);
        *reinterpret_cast<uint4 *>(out + c * 8) = o;
    }
}

}  // namespace

hipError_t launch_smooth_fold(const uint16_t *w, int dtype, int64_t N, int64_t K,
                              const float *smooth, uint16_t *w_out, hipStream_t stream)
{
    const int64_t chunks = N * K / 8;
    if (chunks == 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 4096);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL((smooth_fold_kernel<DT_BF16>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           w, N, K, smooth, w_out);
    else
        hipLaunchKernelGGL((smooth_fold_kernel<DT_F16>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           w, N, K, smooth, w_out);
    return hipGetLastError();
}

}  // namespace cider
