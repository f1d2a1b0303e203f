// Row-wise symmetric quantization kernels: per-token activations (Cider
// README, ossradar.top repo page, "Metal Kernel Pipeline": FP16 activations
// -> INT8 + per-token scales) and the offline weight quantizers ("Low-Level
// API": quantize_weight_int8, pack_weight_int4; "W8A8 Quantization
// Granularity": per channel or per group of 64 / 128).
//
// A "team" of TS lanes owns one row: it loads the row once in 16-byte
// chunks (8 fp16 per lane per chunk, adjacent lanes adjacent in memory),
// keeps it in registers, reduces the absmax with cross-lane shuffles (a
// whole-workgroup team also through LDS), then writes the codes (8 bytes or
// 4 packed bytes per chunk, again contiguous across lanes) and the scale.
// Short rows (weight groups of 64 / 128) use teams of 8 / 16 lanes so a
// wavefront still covers 512 bytes per load; long rows use teams of 64 or,
// when few or very long, of 256 lanes.
// Rows longer than the register budget take a two-pass kernel that re-reads
// the row from cache.
//
// Inputs are fp16 or bf16 (README feature list: fp16 / bf16 dtype handling),
// widened exactly.  Activations may carry a SmoothQuant smoothing vector
// (README: SmoothQuant named as the preprocessing that makes activations
// quantization-friendly): each element is divided by its channel's factor
// (correctly rounded fp32 quotient) before the absmax, and the quotients are
// what gets quantized; the factors are re-read per chunk (cache hits: every
// row uses the same K factors).
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

// Smoothing factors of the 8 elements at chunk c (k = 8c .. 8c+7).
__device__ __forceinline__ void load_smooth(const float *__restrict__ sm, int64_t c, float (&f)[8])
{
    const float4 a = *reinterpret_cast<const float4 *>(sm + c * 8);
    const float4 b = *reinterpret_cast<const float4 *>(sm + c * 8 + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Magnitude bits of the largest |value| of a chunk.  Without smoothing: the
// 16-bit elements' own magnitude bits; with it: the fp32 quotients' bits
// (for finite values both orders are the value order).
template <int DT, bool SMOOTH>
__device__ __forceinline__ uint32_t chunk_amax(uint4 v, const float *__restrict__ sm, int64_t c)
{
    if constexpr (!SMOOTH) {
        return chunk_absmax_bits(v);
    } else {
        float l[8], f[8];
        load_smooth(sm, c, l);
        smooth_chunk<DT>(v, l, f);
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = __builtin_bit_cast(uint32_t, f[e]) & 0x7FFFFFFFu;
            m = b > m ? b : m;
        }
        return m;
    }
}

template <int DT, bool SMOOTH>
__device__ __forceinline__ float amax_value(uint32_t bits)
{
    if constexpr (SMOOTH)
        return __builtin_bit_cast(float, bits);
    else
        return widen_bits<DT>(bits);
}

// Codes of a chunk for scale s (rs = 1 / s): the product with rs and the
// exact near-half fallback when the row's chunks fit in registers (FAST),
// else a division per value (fewer live registers for long rows).
template <int BITS, int DT, bool SMOOTH, bool FAST>
__device__ __forceinline__ uint2 chunk_codes(uint4 v, const float *__restrict__ sm, int64_t c, float s,
                                             float rs)
{
    if constexpr (SMOOTH) {
        float l[8], f[8];
        load_smooth(sm, c, l);
        smooth_chunk<DT>(v, l, f);
        return quantize_values<BITS>(f, s, rs);
    } else if constexpr (FAST) {
        return quantize_chunk<BITS, DT>(v, s, rs);
    } else {
        return quantize_chunk_div<BITS, DT>(v, s);
    }
}

// The largest magnitude bits over a team of TS lanes (a whole-workgroup team
// also through LDS); every lane of the team gets the result.
template <int TS>
__device__ __forceinline__ uint32_t team_max(uint32_t amax, int lane)
{
    if constexpr (TS <= 64) {
#pragma unroll
        for (int o = TS / 2; o > 0; o >>= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)amax, o, TS);
            amax = other > amax ? other : amax;
        }
    } else {
        __shared__ uint32_t red[TS / 64];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)amax, o, 64);
            amax = other > amax ? other : amax;
        }
        if ((lane & 63) == 0)
            red[lane >> 6] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int w = 1; w < TS / 64; ++w)
            amax = red[w] > amax ? red[w] : amax;
    }
    return amax;
}

// The quantization of one row held by a team of TS lanes in v[0 .. NCH-1]
// (chunk i * TS + lane; lanes past the row end hold a copy of its last chunk,
// masked out here): absmax by shuffles, the scale, the codes, the stores.
// With smoothing and at most 8 chunks per lane, each value's quotient by its
// smoothing factor is computed once and kept for both the absmax and the
// codes (the same divisions, half as many); longer rows recompute it.
template <int TS, int NCH, int BITS, int DT, bool SMOOTH>
__device__ __forceinline__ void quantize_team_row(const uint4 (&v)[NCH], int64_t row, int lane, int nch,
                                                  int64_t len, const float *__restrict__ smooth,
                                                  uint8_t *__restrict__ out, float *__restrict__ scale)
{
    constexpr bool KEEP = SMOOTH && NCH <= 8;
    float fs[KEEP ? NCH : 1][8];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = i * TS + lane;
        uint32_t m;
        if constexpr (KEEP) {
            float l[8];
            load_smooth(smooth, min(c, nch - 1), l);
            smooth_chunk<DT>(v[i], l, fs[i]);
            m = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t b = __builtin_bit_cast(uint32_t, fs[i][e]) & 0x7FFFFFFFu;
                m = b > m ? b : m;
            }
        } else {
            m = chunk_amax<DT, SMOOTH>(v[i], smooth, min(c, nch - 1));
        }
        amax = (c < nch && m > amax) ? m : amax;
    }
    amax = team_max<TS>(amax, lane);
    const float s = amax_value<DT, SMOOTH>(amax) / quant_divisor<BITS>();
    const float rs = 1.0f / s;
    if (lane == 0)
        scale[row] = s;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = i * TS + lane;
        if (c < nch) {
            uint2 q;
            if constexpr (KEEP)
                q = quantize_values<BITS>(fs[i], s, rs);
            else
                q = chunk_codes<BITS, DT, SMOOTH, (NCH <= 8)>(v[i], smooth, c, s, rs);
            if constexpr (BITS == 8)
                *reinterpret_cast<uint2 *>(out + row * len + (int64_t)c * 8) = q;
            else
                *reinterpret_cast<uint32_t *>(out + row * (len / 2) + (int64_t)c * 4) = q.x;
        }
    }
}

// A row's chunks into registers.  Every load is issued before any is used: a
// lane past the row end re-reads the row's last chunk (an address that is
// always valid), so no branch separates the loads (a branch would make the
// compiler wait for each load at the join).  The rows are read once:
// non-temporal loads (5-13% faster on the activation shapes).
template <int TS, int NCH>
__device__ __forceinline__ void load_team_row(const uint16_t *__restrict__ xr, int lane, int nch,
                                              uint4 (&v)[NCH])
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = min(i * TS + lane, nch - 1);
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (int64_t)c * 8));
        v[i] = uint4{t.x, t.y, t.z, t.w};
    }
}

template <int TS, int NCH, int BITS, int DT, bool SMOOTH>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *__restrict__ x,
                                                            int64_t rows, int64_t len, int64_t ld,
                                                            const float *__restrict__ smooth,
                                                            uint8_t *__restrict__ out,
                                                            float *__restrict__ scale,
                                                            uint32_t *__restrict__ zero, int nzero)
{
    constexpr int TEAMS = 256 / TS;
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < nzero; i += 256)
            zero[i] = 0u;
    const int lane = threadIdx.x % TS;
    const int64_t row = (int64_t)blockIdx.x * TEAMS + threadIdx.x / TS;
    if (row >= rows)
        return;  // a team is part of one wavefront or the whole workgroup: whole teams
                 // leave together (a 256-lane team's LDS barrier is reached by all or none)
    const int nch = (int)(len >> 3);
    uint4 v[NCH];
    load_team_row<TS, NCH>(x + row * ld, lane, nch, v);
    quantize_team_row<TS, NCH, BITS, DT, SMOOTH>(v, row, lane, nch, len, smooth, out, scale);
}

// One workgroup per row, any length: absmax pass, then a quantize pass that
// reads the row again.
template <int BITS, int DT, bool SMOOTH>
__global__ __launch_bounds__(256) void quantize_long_rows_kernel(const uint16_t *__restrict__ x,
                                                                 int64_t len, int64_t ld,
                                                                 const float *__restrict__ smooth,
                                                                 uint8_t *__restrict__ out,
                                                                 float *__restrict__ scale,
                                                                 uint32_t *__restrict__ zero, int nzero)
{
    __shared__ uint32_t red[4];
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < nzero; i += 256)
            zero[i] = 0u;
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * ld;
    const int64_t nch = len >> 3;
    uint32_t amax = 0;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint32_t m = chunk_amax<DT, SMOOTH>(*reinterpret_cast<const uint4 *>(xr + c * 8), smooth, c);
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
    const float s = amax_value<DT, SMOOTH>(amax) / quant_divisor<BITS>();
    const float rs = 1.0f / s;
    if (threadIdx.x == 0)
        scale[row] = s;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const uint2 q = chunk_codes<BITS, DT, SMOOTH, true>(*reinterpret_cast<const uint4 *>(xr + c * 8),
                                                            smooth, c, s, rs);
        if constexpr (BITS == 8)
            *reinterpret_cast<uint2 *>(out + row * len + c * 8) = q;
        else
            *reinterpret_cast<uint32_t *>(out + row * (len / 2) + c * 4) = q.x;
    }
}

template <int TS, int NCH, int BITS, int DT, bool SMOOTH>
hipError_t launch_team(const uint16_t *x, int64_t rows, int64_t len, int64_t ld, const float *smooth,
                       void *out, float *scale, hipStream_t stream, uint32_t *zero, int nzero)
{
    constexpr int TEAMS = 256 / TS;
    const int64_t blocks = (rows + TEAMS - 1) / TEAMS;
    hipLaunchKernelGGL((quantize_rows_kernel<TS, NCH, BITS, DT, SMOOTH>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, x, rows, len, ld, smooth, static_cast<uint8_t *>(out),
                       scale, zero, nzero);
    return hipGetLastError();
}

template <int BITS, int DT, bool SMOOTH>
hipError_t launch_bits(const uint16_t *x, int64_t rows, int64_t len, int64_t ld, const float *smooth,
                       void *out, float *scale, hipStream_t stream, uint32_t *zero, int nzero)
{
    const int64_t nch = len / 8;
    if (nch <= 8)
        return launch_team<8, 1, BITS, DT, SMOOTH>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
    if (nch <= 16)
        return launch_team<16, 1, BITS, DT, SMOOTH>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
    if (nch <= 32)
        return launch_team<32, 1, BITS, DT, SMOOTH>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
    // Rows of more than 256 chunks, when there are few of them (up to 512)
    // or they are long (1024 chunks and more): a whole workgroup per row, so
    // each lane holds at most 8 chunks and the row's loads and codes spread
    // over 4 wavefronts (K = 10240: M = 16 8.2 -> 3.9 us, M = 4096 35.8 ->
    // 27.3 us; at K = 2560 and thousands of rows a wavefront per row stays
    // faster).
    if (nch > 256 && nch <= 256 * 8 && (rows <= 512 || nch >= 1024)) {
        const int64_t pl = (nch + 255) / 256;
#define CIDER_TEAM256(n)                                                                         \
    if (pl <= n)                                                                                 \
        return launch_team<256, n, BITS, DT, SMOOTH>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
        CIDER_TEAM256(2)
        CIDER_TEAM256(3)
        CIDER_TEAM256(4)
        CIDER_TEAM256(5)
        CIDER_TEAM256(6)
        CIDER_TEAM256(8)
#undef CIDER_TEAM256
    }
    const int64_t per_lane = (nch + 63) / 64;
#define CIDER_TEAM64(n)                                                                          \
    if (per_lane <= n)                                                                           \
        return launch_team<64, n, BITS, DT, SMOOTH>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
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
    hipLaunchKernelGGL((quantize_long_rows_kernel<BITS, DT, SMOOTH>), dim3((unsigned)rows), dim3(256),
                       0, stream, x, len, ld, smooth, static_cast<uint8_t *>(out), scale, zero, nzero);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int dtype, int64_t rows, int64_t len, int64_t ld,
                                const float *smooth, int bits, void *out, float *scale,
                                hipStream_t stream, uint32_t *zero, int nzero)
{
    if (rows == 0)
        return hipSuccess;
    if (smooth) {  // activations only: int8 codes
        if (bits != 8)
            return hipErrorInvalidValue;
        return dtype == DT_BF16 ? launch_bits<8, DT_BF16, true>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero)
                                : launch_bits<8, DT_F16, true>(x, rows, len, ld, smooth, out, scale, stream, zero, nzero);
    }
    if (dtype == DT_BF16)
        return bits == 8 ? launch_bits<8, DT_BF16, false>(x, rows, len, ld, nullptr, out, scale, stream, zero, nzero)
                         : launch_bits<4, DT_BF16, false>(x, rows, len, ld, nullptr, out, scale, stream, zero, nzero);
    return bits == 8 ? launch_bits<8, DT_F16, false>(x, rows, len, ld, nullptr, out, scale, stream, zero, nzero)
                     : launch_bits<4, DT_F16, false>(x, rows, len, ld, nullptr, out, scale, stream, zero, nzero);
}

}  // namespace cider
