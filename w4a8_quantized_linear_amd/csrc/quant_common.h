// Device-side quantization arithmetic shared by the quantize kernels and the
// fused one-token matrix-vector kernel, so all produce identical codes.
//
// Cider README (ossradar.top repo page), "Quantization" table: symmetric INT8
// per token for activations, symmetric INT8 / INT4 (zero-point 8) for weights.
// Scale s = absmax / 127 (or / 7), code q = clamp(rint(x / s)).  Both
// divisions are correctly rounded fp32 divisions (the default HIP lowering;
// the library is never built with fast-math or approximate division) and
// rint rounds half to even (v_rndne_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cider {

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Element types of the fp16 / bf16 inputs.
enum { DT_F16 = 0, DT_BF16 = 1 };

// Exact fp32 value of a 16-bit element (bf16 is the upper half of an fp32).
template <int DT>
__device__ __forceinline__ float widen_bits(uint32_t h)
{
    if constexpr (DT == DT_BF16)
        return __builtin_bit_cast(float, (h & 0xFFFFu) << 16);
    else
        return half_bits_to_float(h & 0xFFFFu);
}

// Largest magnitude among the 8 fp16 (or bf16) values of a 16-byte chunk, as
// magnitude bits.  For finite inputs of either type the order of |x| equals
// the order of the bit patterns with the sign bit cleared.
__device__ __forceinline__ uint32_t chunk_absmax_bits(uint4 v)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu,
                           v.w & 0x7FFF7FFFu};
    u16x2 m = __builtin_bit_cast(u16x2, w[0]);
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[1]));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[2]));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[3]));
    return m.x > m.y ? m.x : m.y;
}

template <int BITS>
__device__ __forceinline__ float quant_divisor()
{
    return BITS == 8 ? 127.0f : 7.0f;
}

// Integer code of x for scale s, given the quotient x / s.  Branch-free: for
// s == 0 (an all-zero row) the quotient is discarded by the final select.
template <int BITS>
__device__ __forceinline__ int code_of(float quotient, float s)
{
    constexpr float lo = BITS == 8 ? -127.0f : -8.0f;
    constexpr float hi = BITS == 8 ? 127.0f : 7.0f;
    float r = __builtin_rintf(quotient);
    r = __builtin_fminf(__builtin_fmaxf(r, lo), hi);  // maxNum/minNum: NaN -> bound
    return s == 0.0f ? 0 : (int)r;
}

// Packs 8 codes: int8 -> 8 bytes (uint2), int4 -> 8 nibbles u = q + 8 with
// value e at bits 4e (uint32 in .x).
template <int BITS>
__device__ __forceinline__ uint2 pack_codes(const int (&q)[8])
{
    uint2 o;
    if constexpr (BITS == 8) {
        o.x = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
              ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
        o.y = (uint32_t)(q[4] & 0xFF) | ((uint32_t)(q[5] & 0xFF) << 8) |
              ((uint32_t)(q[6] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
    } else {
        uint32_t p = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            p |= (uint32_t)(q[e] + 8) << (4 * e);
        o.x = p;
        o.y = 0;
    }
    return o;
}

// True when the scale is not a normal fp32 number (below 2^-126: bf16 rows
// with absmax below about 1.5e-36, rows divided by huge smoothing factors).
// Below 2^-128 the reciprocal rs = 1 / s overflows to +inf, so x * rs is
// +-inf, or NaN for x = 0, and cannot stand in for the quotient x / s; the
// bound on the product's error below is stated for normal scales only, so
// every row under 2^-126 takes the correctly rounded division for every
// value.  All-zero rows (s == 0) take it too; their codes are 0 either way.
__device__ __forceinline__ bool tiny_scale(float s)
{
    return !(s >= 0x1p-126f);
}

// Codes of the 8 fp16 values of a chunk, packed: int8 -> 8 bytes (uint2),
// int4 -> 8 nibbles u = q + 8 with value e at bits 4e (uint32 in .x).
// rs must be 1.0f / s (correctly rounded).
//
// The code is rint of the correctly rounded quotient fl(x / s).  For a normal
// scale s the product t = fl(x * rs) differs from fl(x / s) by at most
// 3 * 2^-24 relative, i.e. below 2^-15.4 in absolute terms for
// |x / s| <= 127.5, so rint(t) equals rint(fl(x / s)) unless t lies within
// that distance of a half-integer.  A chunk with a value within 2^-14 of a
// half-integer (about 1 value in 8000), or any chunk of a row whose scale is
// not a normal fp32 (tiny_scale), is recomputed with correctly rounded
// divisions.
template <int BITS, int DT = DT_F16>
__device__ __forceinline__ uint2 quantize_chunk(uint4 v, float s, float rs)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8], t[8];
    bool near_half = tiny_scale(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = widen_bits<DT>(w[j]);
        f[2 * j + 1] = widen_bits<DT>(w[j] >> 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        t[e] = f[e] * rs;
        const float d = t[e] - __builtin_rintf(t[e]);  // in [-0.5, 0.5]; NaN stays unflagged
        near_half |= __builtin_fabsf(__builtin_fabsf(d) - 0.5f) < 0x1p-14f;
    }
    if (near_half) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            t[e] = f[e] / s;
    }
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        q[e] = code_of<BITS>(t[e], s);
    return pack_codes<BITS>(q);
}

// The same codes with a correctly rounded division for every value (fewer
// live registers: for kernels that hold long rows in registers).
template <int BITS, int DT = DT_F16>
__device__ __forceinline__ uint2 quantize_chunk_div(uint4 v, float s)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    int q[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[2 * j] = code_of<BITS>(widen_bits<DT>(w[j]) / s, s);
        q[2 * j + 1] = code_of<BITS>(widen_bits<DT>(w[j] >> 16) / s, s);
    }
    return pack_codes<BITS>(q);
}

// Smoothed values of a chunk: the 8 elements at k .. k+7 divided by their
// smoothing factors sm[0..7] (correctly rounded fp32 quotients).
template <int DT>
__device__ __forceinline__ void smooth_chunk(uint4 v, const float (&sm)[8], float (&f)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = widen_bits<DT>(w[j]) / sm[2 * j];
        f[2 * j + 1] = widen_bits<DT>(w[j] >> 16) / sm[2 * j + 1];
    }
}

// Codes of 8 fp32 values, packed: rint of the correctly rounded quotients by
// s, through the product with rs = 1 / s and the same near-half and tiny-scale
// fallbacks as quantize_chunk.  (fp32 values, so the bound on |f / s| is 127.5
// again: the scale comes from their own absmax.)
template <int BITS>
__device__ __forceinline__ uint2 quantize_values(const float (&f)[8], float s, float rs)
{
    float t[8];
    bool near_half = tiny_scale(s);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        t[e] = f[e] * rs;
        const float d = t[e] - __builtin_rintf(t[e]);
        near_half |= __builtin_fabsf(__builtin_fabsf(d) - 0.5f) < 0x1p-14f;
    }
    if (near_half) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            t[e] = f[e] / s;
    }
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        q[e] = code_of<BITS>(t[e], s);
    return pack_codes<BITS>(q);
}

}  // namespace cider
