// Internal launch interface between the C ABI (api.hip) and the gfx950
// kernels.  Arguments arrive here already validated: sizes inside the
// envelope documented in include/cider.h, pointers non-null and aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cider {

// Symmetric absmax quantization of `rows` rows of `len` fp16 (dtype 0) or
// bf16 (dtype 1) values (row stride `ld` elements).  bits 8: out int8
// [rows, len]; bits 4: out uint8 [rows, len/2] packed nibbles.  scale fp32
// [rows].  len % 8 == 0.  smooth (fp32 [len], 16-byte aligned, bits 8 only)
// or null: each element divided by its column's factor before the absmax.
// Per-token activations are rows = M, len = K; per-channel weights rows = N;
// per-group weights are the [N * K/gs, gs] view of W.  `zero` (nzero
// words, or null) is cleared by the same launch: the split product's tile
// counters, reset before every product that uses them.
hipError_t launch_quantize_rows(const uint16_t *x, int dtype, int64_t rows, int64_t len, int64_t ld,
                                const float *smooth, int bits, void *out, float *scale,
                                hipStream_t stream, uint32_t *zero = nullptr, int nzero = 0);

// The same with each row's range the percentile of its |w| (percentile
// clipping): ranks r0 <= r1 of the two order statistics and the
// interpolation weight g, computed by the caller.  len % 8 == 0, len < 2^31.
hipError_t launch_clip_quantize_rows(const uint16_t *w, int dtype, int64_t rows, int64_t len,
                                     int64_t r0, int64_t r1, double g, int bits, void *out,
                                     float *scale, hipStream_t stream);

// SmoothQuant's offline weight fold: w_out[n, k] = w[n, k] * smooth[k], the
// exact product rounded once (to nearest even) to the weight's type.
hipError_t launch_smooth_fold(const uint16_t *w, int dtype, int64_t N, int64_t K,
                              const float *smooth, uint16_t *w_out, hipStream_t stream);

// Output of the product kernels: fp16 or bf16 results, or the raw int32
// accumulators (test hook).
enum OutKind { OUT_F16 = 0, OUT_I32 = 1, OUT_BF16 = 2 };

// Bit pattern of an fp32 result rounded to the output type, to nearest even,
// by the hardware conversion of each type (gfx950 converts to bf16 in one
// instruction; NaN stays a quiet NaN).
template <int OUT>
__device__ __forceinline__ uint16_t out_bits(float y)
{
    if constexpr (OUT == OUT_BF16)
        return __builtin_bit_cast(uint16_t, (__bf16)y);
    else
        return __builtin_bit_cast(uint16_t, (_Float16)y);
}

// Two outputs packed into one dword (first in the low half) by the packed
// hardware conversion of the output type (round to nearest even, as the
// scalar one in out_bits).
template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    if constexpr (OUT == OUT_F16) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
    } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
    }
}

struct ProductArgs {
    const int8_t *xq;      // [M, K]
    const float *s_tok;    // [M]         (OUT_F16)
    const void *wq;        // int8 [N, K] or packed uint8 [N, K/2]
    const float *s_w;      // [N] or [N, K/gs] (OUT_F16)
    int64_t M, N, K;
    int bits;              // 8 or 4
    int group_size;        // 0, 64 or 128
    OutKind out_kind;
    void *out;             // fp16 [M, N] or int32 [M, N] / [M, N, K/gs]
};

// Split-K state handed to the product kernel (all zero: no split).
struct SplitArgs {
    void *part;      // partial sums, [tiles][splits][TM * TN] 4-byte words
    uint32_t *cnt;   // [tiles] arrival counters, zero at launch
    int splits;
};

// Matrix-core product (any M >= 1, every mode); up to 32 tokens it goes to
// the few-token kernel where that supports the shape, else per group with
// M <= 256 to the skinny kernel.
hipError_t launch_gemm(const ProductArgs &a, hipStream_t stream);

// Split-K product for few tokens (fp16 / bf16 output only).  Each output
// tile is computed by `splits` workgroups over disjoint K ranges (whole
// groups per group); each writes its partial sums (int32 per channel, the
// group-scaled fp32 sums per group) to `part`, and the last one to finish
// (counted in cnt[tile], which must be zero at launch) adds them up in split
// order and stores the dequantized tile.
struct SplitPlan {
    int splits;          // 1: no split
    int64_t tiles;       // output tiles = counters
    int64_t tile_elems;  // partial-sum words per tile and split
};
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int bits, int group_size);
hipError_t launch_gemm_split(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream);
hipError_t launch_gemm_skinny(const ProductArgs &a, hipStream_t stream);

// Few-token product (every mode but the per-group int32 hook; K a multiple of
// 128 for int8 weights, 256 for int4): weights streamed as whole lines and
// turned into matrix-core operands in per-wavefront LDS slots, 16 or 32
// tokens per tile.  few_shape_ok: the kernel can take the shape at any M;
// few_supported: it is the product of choice (M <= 32).  launch_gemm_few
// takes any shape few_shape_ok accepts.
bool few_shape_ok(const ProductArgs &a);
bool few_supported(const ProductArgs &a);
hipError_t launch_gemm_few(const ProductArgs &a, hipStream_t stream);

// Matrix-vector product for M <= 8 and M * K <= 32768.
hipError_t launch_gemv(const ProductArgs &a, hipStream_t stream);

// Few-token layer on the matrix-vector path: quantizes the fp16 rows x [M, K]
// (row stride ldx elements, M <= 8) inside the matrix-vector kernel and
// writes y [M, N] (fp16 or bf16 by out_kind).  xq_out [M, K] / s_tok_out [M]
// may be null; when given, the quantized rows and their scales are written
// there as well.
hipError_t launch_gemv_fused(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const void *wq,
                             const float *s_w, int64_t N, int bits, int group_size, void *y,
                             int8_t *xq_out, float *s_tok_out, int out_kind, hipStream_t stream);

// The decode variant (no activation quantization): y [N] = fp16 / bf16 of
// sum_g s_w[n, g] * sum_{k in g} x[k] * q[n, k], x fp16 [K] (16-byte aligned),
// K % 64 == 0, K <= 16384 (int8) or 32768 (int4).
hipError_t launch_decode(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                         int bits, int group_size, int out_kind, void *y, hipStream_t stream);

}  // namespace cider
