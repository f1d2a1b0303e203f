// Matrix-vector product for one (up to 8) token(s): the decode path of the
// layer (Cider README, ossradar.top repo page, "Metal Kernel Pipeline",
// Decode (M = 1): int8_mv; "Quick Start": seq_len == 1 -> INT8 MV kernel).
// The pages' decode kernel skips activation quantization; this one computes
// the same W8A8 / W4A8 function as the matrix-core kernel at every M, so a
// one-token call and a batched call agree.
//
// The work is a stream of the weight matrix from HBM: each wavefront owns
// ROWS weight rows at a time, every lane loads 16-byte chunks of those rows
// (adjacent lanes adjacent in memory, several chunks in flight per lane),
// multiplies them against the token's int8 codes held in LDS with
// v_dot4_i32_i8, and the wavefront reduces the exact int32 sum with
// cross-lane shuffles.  Per-group scaling first reduces each group's int32
// sum across the lanes that hold it (4 or 8 lanes), then scales it.
//
// Fused variant (one fp16 token): every workgroup reads the whole row (a few
// KB, served from L2 after the first workgroup), reduces its absmax,
// quantizes it into LDS with the same arithmetic as the quantize kernel, and
// only then streams its weight rows; no second launch and no int8 round trip
// through memory.
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 2;
constexpr int kUnroll = 4;  // chunks per lane loaded before use

__device__ __forceinline__ int dot16(uint4 w, uint4 x, int acc)
{
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
    return acc;
}

__device__ __forceinline__ void unpack8(uint32_t v, uint32_t &d0, uint32_t &d1)
{
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    const uint32_t a = (lo & 0xFFu) | ((hi & 0xFFu) << 8) | ((lo & 0xFF00u) << 8) | ((hi & 0xFF00u) << 16);
    const uint32_t b = ((lo >> 16) & 0xFFu) | ((hi >> 8) & 0xFF00u) | ((lo & 0xFF000000u) >> 8) |
                       (hi & 0xFF000000u);
    d0 = (a + 0x78787878u) ^ 0x80808080u;
    d1 = (b + 0x78787878u) ^ 0x80808080u;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

struct GemvParams {
    const int8_t *xq;       // [M, K] (unused when fused)
    const uint16_t *x;      // fp16 [K] (fused only)
    const float *s_tok;     // [M] (unused when fused)
    const uint8_t *wq;      // int8 [N, K] or packed [N, K/2]
    const float *s_w;       // [N] or [N, G]
    int64_t M, N, K;
    void *out;
    int8_t *xq_out;         // fused: optional copy of the codes
    float *s_tok_out;       // fused: optional copy of the scale
};

// BITS 8 or 4; GS 0 / 64 / 128; OUT fp16 or int32; FUSED quantizes x first.
template <int BITS, int GS, int OUT, bool FUSED>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t sx[];  // [M][K] int8 codes
    __shared__ float s_red[kWaves];
    __shared__ uint32_t u_red[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int G = GS ? (int)(K / GS) : 1;

    float s_tok_fused = 0.f;
    if constexpr (FUSED) {
        const int64_t nch = K >> 3;
        uint32_t amax = 0;
        for (int64_t c = tid; c < nch; c += kThreads) {
            const uint32_t m = chunk_absmax_bits(*reinterpret_cast<const uint4 *>(p.x + c * 8));
            amax = m > amax ? m : amax;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)amax, o, 64);
            amax = other > amax ? other : amax;
        }
        if (lane == 0)
            u_red[wave] = amax;
        __syncthreads();
        amax = u_red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            amax = u_red[w] > amax ? u_red[w] : amax;
        const float s = half_bits_to_float(amax) / quant_divisor<8>();
        s_tok_fused = s;
        for (int64_t c = tid; c < nch; c += kThreads) {
            const uint2 q = quantize_chunk<8>(*reinterpret_cast<const uint4 *>(p.x + c * 8), s);
            *reinterpret_cast<uint2 *>(sx + c * 8) = q;
            if (blockIdx.x == 0 && p.xq_out)
                *reinterpret_cast<uint2 *>(p.xq_out + c * 8) = q;
        }
        if (blockIdx.x == 0 && tid == 0 && p.s_tok_out)
            p.s_tok_out[0] = s;
    } else {
        const int64_t nch = (M * K) >> 4;
        for (int64_t c = tid; c < nch; c += kThreads)
            *reinterpret_cast<uint4 *>(sx + c * 16) = *reinterpret_cast<const uint4 *>(p.xq + c * 16);
    }
    __syncthreads();

    // Chunks of 16 weight bytes per row: int8 -> 16 k values, int4 -> 32.
    constexpr int KPC = BITS == 8 ? 16 : 32;
    const int64_t nch = K / KPC;
    const int64_t wld = BITS == 8 ? K : K / 2;
    const int64_t rows_per_block = (int64_t)kWaves * kRowsPerWave;
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_block + wave * kRowsPerWave;

    for (int64_t m = 0; m < M; ++m) {
        const uint8_t *xm = sx + m * K;
        int iacc[kRowsPerWave];
        float facc[kRowsPerWave];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            iacc[r] = 0;
            facc[r] = 0.f;
        }
        for (int64_t c0 = 0; c0 < nch; c0 += 64 * kUnroll) {
            uint4 wv[kRowsPerWave][kUnroll];
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
                const int64_t n = min(row0 + r, N - 1);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t c = c0 + u * 64 + lane;
                    wv[r][u] = c < nch ? *reinterpret_cast<const uint4 *>(p.wq + n * wld + c * 16)
                                       : uint4{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t c = c0 + u * 64 + lane;
                const bool live = c < nch;
                const int64_t cc = live ? c : 0;
                uint4 xa = *reinterpret_cast<const uint4 *>(xm + cc * KPC);
                uint4 xb = uint4{0, 0, 0, 0};
                if constexpr (BITS == 4)
                    xb = *reinterpret_cast<const uint4 *>(xm + cc * KPC + 16);
#pragma unroll
                for (int r = 0; r < kRowsPerWave; ++r) {
                    int d;
                    if constexpr (BITS == 8) {
                        d = dot16(wv[r][u], xa, 0);
                    } else {
                        uint4 lo, hi;
                        unpack8(wv[r][u].x, lo.x, lo.y);
                        unpack8(wv[r][u].y, lo.z, lo.w);
                        unpack8(wv[r][u].z, hi.x, hi.y);
                        unpack8(wv[r][u].w, hi.z, hi.w);
                        d = dot16(hi, xb, dot16(lo, xa, 0));
                    }
                    d = live ? d : 0;
                    if constexpr (GS == 0) {
                        iacc[r] += d;
                    } else {
                        // lanes 4g..4g+3 (gs 64) or 8g..8g+7 (gs 128) hold one group
                        constexpr int LPG = GS / KPC;
#pragma unroll
                        for (int o = 1; o < LPG; o <<= 1)
                            d += __shfl_xor(d, o, 64);
                        const int64_t n = row0 + r;
                        if ((lane & (LPG - 1)) == 0 && live && n < N) {
                            const int64_t g = (c * KPC) / GS;
                            if constexpr (OUT == OUT_I32)
                                static_cast<int32_t *>(p.out)[(m * N + n) * G + g] = d;
                            else
                                facc[r] += (float)d * p.s_w[n * G + g];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            const int64_t n = row0 + r;
            if constexpr (GS == 0) {
                const int total = wave_sum(iacc[r]);
                if (lane == 0 && n < N) {
                    if constexpr (OUT == OUT_I32) {
                        static_cast<int32_t *>(p.out)[m * N + n] = total;
                    } else {
                        const float st = FUSED ? s_tok_fused : p.s_tok[m];
                        const float y = (float)total * st * p.s_w[n];
                        static_cast<uint16_t *>(p.out)[m * N + n] =
                            __builtin_bit_cast(uint16_t, (_Float16)y);
                    }
                }
            } else if constexpr (OUT == OUT_F16) {
                const float t = wave_sum(facc[r]);
                if (lane == 0 && n < N) {
                    const float st = FUSED ? s_tok_fused : p.s_tok[m];
                    static_cast<uint16_t *>(p.out)[m * N + n] =
                        __builtin_bit_cast(uint16_t, (_Float16)(st * t));
                }
            }
        }
    }
    (void)s_red;
}

template <int BITS, int GS, int OUT, bool FUSED>
hipError_t launch_one(const GemvParams &p, hipStream_t stream)
{
    const int64_t rows_per_block = (int64_t)kWaves * kRowsPerWave;
    const int64_t blocks = (p.N + rows_per_block - 1) / rows_per_block;
    const size_t lds = (size_t)(FUSED ? 1 : p.M) * (size_t)p.K;
    hipLaunchKernelGGL((gemv_kernel<BITS, GS, OUT, FUSED>), dim3((unsigned)blocks), dim3(kThreads),
                       lds, stream, p);
    return hipGetLastError();
}

template <int OUT, bool FUSED>
hipError_t dispatch(const GemvParams &p, int bits, int group_size, hipStream_t stream)
{
    if (bits == 8) {
        switch (group_size) {
        case 0: return launch_one<8, 0, OUT, FUSED>(p, stream);
        case 64: return launch_one<8, 64, OUT, FUSED>(p, stream);
        case 128: return launch_one<8, 128, OUT, FUSED>(p, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (group_size == 0)
        return launch_one<4, 0, OUT, FUSED>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const ProductArgs &a, hipStream_t stream)
{
    GemvParams p{};
    p.xq = a.xq;
    p.s_tok = a.s_tok;
    p.wq = static_cast<const uint8_t *>(a.wq);
    p.s_w = a.s_w;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.out = a.out;
    if (a.out_kind == OUT_F16)
        return dispatch<OUT_F16, false>(p, a.bits, a.group_size, stream);
    return dispatch<OUT_I32, false>(p, a.bits, a.group_size, stream);
}

hipError_t launch_gemv_fused(const uint16_t *x, int64_t K, const void *wq, const float *s_w,
                             int64_t N, int bits, int group_size, void *y, int8_t *xq_out,
                             float *s_tok_out, hipStream_t stream)
{
    GemvParams p{};
    p.x = x;
    p.wq = static_cast<const uint8_t *>(wq);
    p.s_w = s_w;
    p.M = 1;
    p.N = N;
    p.K = K;
    p.out = y;
    p.xq_out = xq_out;
    p.s_tok_out = s_tok_out;
    return dispatch<OUT_F16, true>(p, bits, group_size, stream);
}

}  // namespace cider
