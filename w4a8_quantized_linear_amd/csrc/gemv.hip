// Matrix-vector product for one (up to 8) token(s): the decode path of the
// layer (Cider README, ossradar.top repo page, "Metal Kernel Pipeline",
// Decode (M = 1): int8_mv; "Quick Start": seq_len == 1 -> INT8 MV kernel).
// The pages' decode kernel skips activation quantization; this one computes
// the same W8A8 / W4A8 function as the matrix-core kernel at every M, so a
// one-token call and a batched call agree.
//
// The work is one pass over the weight matrix, so the kernel is built to keep
// HBM busy:
//   * a workgroup owns R consecutive weight rows (contiguous in memory), split
//     into NSEG K-segments of at most 3 16-byte chunks per lane (a kernel
//     instance with 2 chunk slots when a segment fits in 128 chunks, so no
//     load goes out for a slot no lane uses: int4 one-token calls at K = 2560
//     5.86 -> 5.14 us); the R * NSEG
//     (row, segment) units are dealt round-robin to its 4 (one token) or 8
//     wavefronts, 5 each;
//   * each wavefront loads the token first, then issues the loads of its first
//     two units (adjacent lanes, adjacent 16 bytes); the fused activation
//     quantization (or the copy of the int8 tokens into LDS) runs while they
//     fly, and the remaining units' loads follow, up to 15 per lane in flight;
//   * dot products use v_dot4_i32_i8 against the token codes in LDS; sums are
//     reduced across lanes with DPP row operations and cross-row readlanes;
//   * int4 weights are not re-interleaved: the low nibbles of a 32-bit word
//     (even k) and the high nibbles (odd k) are masked out as unsigned bytes
//     u = q + 8 and dotted with the token codes stored in LDS as, per block of
//     32 k, the 16 even-k codes then the 16 odd-k codes; sum(q x) is then
//     sum(u x) - 8 sum(x), with sum(x) taken once per token (per group: once
//     per token and group);
//   * per-group scaling reduces each group's exact int32 sum over the 4 or 8
//     lanes that hold it before scaling it; per-channel keeps int32 to the end;
//   * each unit's sum goes to LDS, and one thread per output adds a row's
//     segments in segment order (results do not depend on timing).
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

// Threads per workgroup: 256 for one fused token (4-5% faster per call at
// the per-group and int4 shapes than 512), 512 otherwise (the token data of
// up to M * K = 65536 codes spread over more threads' registers).
constexpr int threads_for(int fused) { return fused == 1 ? 256 : 512; }
constexpr int kMaxWaves = 8;
constexpr int kMaxM = 8;
constexpr int kMaxUnitsPerWave = 5;
constexpr int kMaxChunksPerLane = 3;  // per unit: SEG <= 192 (an instance with 2 serves SEG <= 128)
constexpr int kEarlyUnits = 2;        // units whose loads go out before the token is quantized
constexpr int kMaxGroupSums = 1024;   // int4 per group: (token, group) sums of the token codes
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor: raw 32-bit dwords, range-checked
constexpr uint32_t kDead = 0x80000000u;  // an offset past every buffer: the load returns zero

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The weights stream through once: non-temporal loads (the nt cache policy
// bit), measured 7-11% faster per call than loads that allocate normally.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ uint4 load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

struct GemvParams {
    const int8_t *xq;       // [M, K] (unused when fused)
    const uint16_t *x;      // fp16 [K] (fused only)
    const float *s_tok;     // [M] (unused when fused)
    const uint8_t *wq;      // int8 [N, K] or packed [N, K/2]
    const float *s_w;       // [N] or [N, G]
    int64_t M, N, K;
    int64_t ldx;            // fused: row stride of x in elements
    int R, NSEG, SEG;       // rows per workgroup, segments per row, chunks per segment
    void *out;
    int8_t *xq_out;         // fused: optional copy of the codes
    float *s_tok_out;       // fused: optional copy of the scale
};

__device__ __forceinline__ int dot16(uint4 w, uint4 x, int acc)
{
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
    return acc;
}

// DPP lane exchanges within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over aligned groups of L lanes (L = 2, 4, 8 or 16); every lane of a
// group ends with the group's sum.
template <int L>
__device__ __forceinline__ int group_sum(int v)
{
    v += dpp<kXor1>(v);
    if constexpr (L >= 4)
        v += dpp<kXor2>(v);
    if constexpr (L >= 8)
        v += dpp<kHalfMirror>(v);
    if constexpr (L >= 16)
        v += dpp<kMirror>(v);
    return v;
}

// Sum over the whole wavefront, result uniform.
__device__ __forceinline__ int wave_sum_i32(int v)
{
    v = group_sum<16>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ float wave_sum_f32(float v)
{
    int b = __builtin_bit_cast(int, v);
    float t = v + __builtin_bit_cast(float, dpp<kXor1>(b));
    t = t + __builtin_bit_cast(float, dpp<kXor2>(__builtin_bit_cast(int, t)));
    t = t + __builtin_bit_cast(float, dpp<kHalfMirror>(__builtin_bit_cast(int, t)));
    t = t + __builtin_bit_cast(float, dpp<kMirror>(__builtin_bit_cast(int, t)));
    const int tb = __builtin_bit_cast(int, t);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(tb, 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(tb, 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(tb, 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(tb, 48));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    int b = (int)v;
    b = max((unsigned)b, (unsigned)dpp<kXor1>(b));
    b = max((unsigned)b, (unsigned)dpp<kXor2>(b));
    b = max((unsigned)b, (unsigned)dpp<kHalfMirror>(b));
    b = max((unsigned)b, (unsigned)dpp<kMirror>(b));
    const uint32_t a0 = (uint32_t)__builtin_amdgcn_readlane(b, 0), a1 = (uint32_t)__builtin_amdgcn_readlane(b, 16);
    const uint32_t a2 = (uint32_t)__builtin_amdgcn_readlane(b, 32), a3 = (uint32_t)__builtin_amdgcn_readlane(b, 48);
    return max(max(a0, a1), max(a2, a3));
}

// Byte selectors for v_perm_b32 over the 8 bytes {hi:lo}: the even bytes
// (0, 2, 4, 6) and the odd bytes (1, 3, 5, 7).
constexpr uint32_t kEvenBytes = 0x06040200u;
constexpr uint32_t kOddBytes = 0x07050301u;

// BITS 8 or 4; GS 0 / 64 / 128; OUT fp16 or int32; FUSED 0: int8 tokens
// given, 1: one fp16 token quantized first, 2: up to kMaxM fp16 tokens
// quantized first (row stride ldx); XR 16-byte token chunks per thread cover
// the whole token data.
template <int BITS, int GS, int OUT, int FUSED, int XR, int SC>
__global__ __launch_bounds__(threads_for(FUSED)) void gemv_kernel(GemvParams p)
{
    constexpr int kThreads = threads_for(FUSED);
    constexpr int kWaves = kThreads / 64;
    constexpr int KPC = BITS == 8 ? 16 : 32;  // k values per 16-byte weight chunk
    constexpr int LPG = GS ? GS / KPC : 1;    // lanes holding one group (chunks per group)
    constexpr bool kXSum = BITS == 4 && GS == 0;   // the -8 sum(x) correction, per token
    constexpr bool kGXSum = BITS == 4 && GS != 0;  // the same per token and group
    extern __shared__ __attribute__((aligned(16))) uint8_t sx[];  // [M][K] int8 codes
    __shared__ float part[kMaxM * 64];                            // [m][unit] partials
    __shared__ int ipart[kMaxM * 64];
    __shared__ uint32_t red[kMaxWaves];
    __shared__ int xsum[kMaxM];
    __shared__ int xg[kGXSum ? kMaxGroupSums : 1];                // [m][g] group sums of x
    __shared__ uint32_t tmax[kMaxM];                              // FUSED 2: token absmax bits
    __shared__ float stok[kMaxM];                                 // FUSED 2: token scales

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = FUSED == 1 ? 1 : p.M, N = p.N, K = p.K;
    const int R = p.R, NSEG = p.NSEG, SEG = p.SEG;
    const int G = GS ? (int)(K / GS) : 1;
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int64_t wld = BITS == 8 ? K : K / 2;
    const int units = R * NSEG;
    const int64_t KC = K / KPC;
    // Unit u of this wavefront: (wave + 8 u) = row r * NSEG + segment sg.
    auto unit_of = [&](int u, int &r, int &sg) __attribute__((always_inline)) {
        const int unit = wave + u * kWaves;
        r = unit / NSEG;
        sg = unit % NSEG;
        return unit < units;
    };

    // 1. The token's data into registers first: the memory counter is in
    //    order, so anything loaded after the weights would wait for all of
    //    them.  Fused: fp16 chunks of 8 values; otherwise int8 code chunks of
    //    16.  Buffer loads return zeros past the end (no branches, so no
    //    conservative waits at join points).
    const uint32_t xbytes = FUSED == 1   ? (uint32_t)(K * 2)
                            : FUSED == 2 ? (uint32_t)(((M - 1) * p.ldx + K) * 2)
                                         : (uint32_t)(M * K);
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(FUSED ? (void *)p.x : (void *)p.xq, (short)0,
                                                      (int)xbytes, kRsrcWord3);
    uint4 xr[XR];
    // FUSED 2: chunk c (8 values) of the [M, K] tokens is chunk c - tm * KC8
    // of token tm = c / KC8.
    const int KC8 = (int)(K >> 3);
    int tm[FUSED == 2 ? XR : 1];
#pragma unroll
    for (int j = 0; j < XR; ++j) {
        const uint32_t c = (uint32_t)(tid + j * kThreads);
        if constexpr (FUSED == 2) {
            tm[j] = (int)(c / (uint32_t)KC8);
            const bool live = c < (uint32_t)(M * KC8);
            xr[j] = load16(rx, live ? (uint32_t)((tm[j] * p.ldx + (c - tm[j] * KC8) * 8) * 2) : kDead);
        } else {
            xr[j] = load16(rx, c * 16u);
        }
    }

    // 2. The weight loads of this wavefront's first kEarlyUnits units, and the
    //    scales: per group, each chunk's group scale; per channel, the scale
    //    of the one output this thread finishes.  The rest of the weights are
    //    issued once the token codes are in LDS: a wavefront waiting to issue
    //    loads into a full memory queue cannot quantize, and the early units
    //    alone keep enough bytes in flight.
    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)p.wq, (short)0, (int)(N * wld), kRsrcWord3);
    const auto rsw = __builtin_amdgcn_make_buffer_rsrc((void *)p.s_w, (short)0, (int)(N * G * 4), kRsrcWord3);
    uint4 wv[kMaxUnitsPerWave][SC];
    float swv[kMaxUnitsPerWave][SC];
    auto issue = [&](int u) __attribute__((always_inline)) {
        int r, sg;
        const bool valid = unit_of(u, r, sg);
        const uint32_t n = (uint32_t)min(n0 + r, N - 1);  // rows past N: any valid row, never stored
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int c = lane + 64 * i;
            const uint32_t kc = (uint32_t)(sg * SEG + c);
            const bool live = valid && c < SEG && kc < (uint32_t)KC;
            wv[u][i] = load16_stream(rw, live ? n * (uint32_t)wld + kc * 16u : kDead);
            if constexpr (GS != 0 && OUT != OUT_I32)
                swv[u][i] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rsw, live ? (n * G + kc / LPG) * 4u : kDead, 0, 0));
        }
    };
#pragma unroll
    for (int u = 0; u < kEarlyUnits; ++u)
        issue(u);
    const int fin_r = tid % R;  // the output this thread finishes: (tid / R, tid % R)
    const bool fin = tid < M * R && n0 + fin_r < N;
    float fin_sw = 0.f;
    if constexpr (GS == 0 && OUT != OUT_I32)
        fin_sw = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rsw, fin ? (uint32_t)(n0 + fin_r) * 4u : kDead, 0, 0));

    if constexpr ((kXSum && FUSED != 1) || FUSED == 2) {
        if (tid < kMaxM) {
            xsum[tid] = 0;
            tmax[tid] = 0;
        }
        __syncthreads();
    }

    // 3. Token codes into LDS while the weights are in flight.  For int4 the
    //    codes of each block of 32 k are stored even k first, then odd k.
    float s_fused = 0.f;
    if constexpr (FUSED == 2) {
        // Per-token absmax: a wavefront whose 64 chunks belong to one token
        // reduces them first; otherwise each lane adds its chunk's maximum.
        const int nch = (int)(M * KC8);
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int c = tid + j * kThreads;
            const uint32_t mb = c < nch ? chunk_absmax_bits(xr[j]) : 0u;
            const int t0 = __builtin_amdgcn_readfirstlane(tm[j]);
            const int t63 = __builtin_amdgcn_readlane(tm[j], 63);
            if (t0 == t63) {
                const uint32_t w = wave_max_u32(mb);
                if (lane == 0 && t0 < M)
                    atomicMax(&tmax[t0], w);
            } else if (c < nch) {
                atomicMax(&tmax[tm[j]], mb);
            }
        }
        __syncthreads();
        const bool keep = blockIdx.x == 0 && p.xq_out;
        int mprev = -1;
        float s = 0.f, rs = 0.f;
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int c = tid + j * kThreads;
            int csum = 0;
            if (c < nch) {
                const int m = tm[j], cc = c - m * KC8;  // chunk cc of token m
                if (m != mprev) {
                    s = half_bits_to_float(tmax[m]) / quant_divisor<8>();
                    rs = 1.0f / s;
                    mprev = m;
                }
                const uint2 q = quantize_chunk<8>(xr[j], s, rs);
                uint8_t *xm = sx + m * K;
                if constexpr (BITS == 8) {
                    *reinterpret_cast<uint2 *>(xm + cc * 8) = q;
                } else {
                    uint8_t *blk = xm + (cc >> 2) * 32 + (cc & 3) * 4;
                    *reinterpret_cast<uint32_t *>(blk) = __builtin_amdgcn_perm(q.y, q.x, kEvenBytes);
                    *reinterpret_cast<uint32_t *>(blk + 16) = __builtin_amdgcn_perm(q.y, q.x, kOddBytes);
                    csum = __builtin_amdgcn_sdot4((int)q.x, 0x01010101, 0, false);
                    csum = __builtin_amdgcn_sdot4((int)q.y, 0x01010101, csum, false);
                }
                if (cc == 0) {
                    stok[m] = s;
                    if (blockIdx.x == 0 && p.s_tok_out)
                        p.s_tok_out[m] = s;
                }
                if (keep)
                    *reinterpret_cast<uint2 *>(p.xq_out + (int64_t)c * 8) = q;
            }
            if constexpr (kXSum) {
                // the token's code sum (int4 correction), reduced like the absmax
                const int t0 = __builtin_amdgcn_readfirstlane(tm[j]);
                const int t63 = __builtin_amdgcn_readlane(tm[j], 63);
                if (t0 == t63) {
                    const int w = wave_sum_i32(csum);
                    if (lane == 0 && t0 < M)
                        atomicAdd(&xsum[t0], w);
                } else if (c < nch) {
                    atomicAdd(&xsum[tm[j]], csum);
                }
            }
            if constexpr (kGXSum) {
                // the GS / 8 chunks of a (token, group) sit on consecutive lanes
                const int gsum = group_sum<GS / 8>(csum);
                if ((tid & (GS / 8 - 1)) == 0 && c < nch)
                    xg[(c * 8) / GS] = gsum;
            }
        }
    } else if constexpr (FUSED == 1) {
        const int64_t nch = K >> 3;
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const uint32_t m = chunk_absmax_bits(xr[j]);  // zero chunks past the row add nothing
            amax = m > amax ? m : amax;
        }
        amax = wave_max_u32(amax);
        if (lane == 0)
            red[wave] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            amax = red[w] > amax ? red[w] : amax;
        const float s = half_bits_to_float(amax) / quant_divisor<8>();
        const float rs = 1.0f / s;
        s_fused = s;
        const bool keep = blockIdx.x == 0 && p.xq_out;
        int tsum = 0;
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int64_t c = tid + (int64_t)j * kThreads;
            int csum = 0;  // sum of this chunk's codes (int4 weights)
            if (c < nch) {
                const uint2 q = quantize_chunk<8>(xr[j], s, rs);
                if constexpr (BITS == 8) {
                    *reinterpret_cast<uint2 *>(sx + c * 8) = q;
                } else {
                    // chunk c holds k = 8c .. 8c+7: block c / 4, quarter c % 4
                    uint8_t *blk = sx + (c >> 2) * 32 + (c & 3) * 4;
                    *reinterpret_cast<uint32_t *>(blk) = __builtin_amdgcn_perm(q.y, q.x, kEvenBytes);
                    *reinterpret_cast<uint32_t *>(blk + 16) = __builtin_amdgcn_perm(q.y, q.x, kOddBytes);
                    csum = __builtin_amdgcn_sdot4((int)q.x, 0x01010101, 0, false);
                    csum = __builtin_amdgcn_sdot4((int)q.y, 0x01010101, csum, false);
                }
                if (keep)
                    *reinterpret_cast<uint2 *>(p.xq_out + c * 8) = q;
            }
            tsum += csum;
            if constexpr (kGXSum) {
                // the GS / 8 chunks of a group sit on consecutive lanes
                const int gsum = group_sum<GS / 8>(csum);
                if ((tid & (GS / 8 - 1)) == 0 && c < nch)
                    xg[(c * 8) / GS] = gsum;
            }
        }
        if constexpr (kXSum) {
            tsum = wave_sum_i32(tsum);
            if (lane == 0)
                ipart[wave] = tsum;  // read after the barrier below, rewritten only after another
        }
        if (blockIdx.x == 0 && tid == 0 && p.s_tok_out)
            p.s_tok_out[0] = s;
    } else {
        const int64_t nch = (M * K) >> 4;
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int64_t c = tid + (int64_t)j * kThreads;
            int csum = 0;
            if (c < nch) {
                if constexpr (BITS == 8) {
                    *reinterpret_cast<uint4 *>(sx + c * 16) = xr[j];
                } else {
                    // chunk c holds k = 16c .. 16c+15 of its token: block c / 2, half c % 2
                    const uint4 v = xr[j];
                    uint8_t *blk = sx + (c >> 1) * 32 + (c & 1) * 8;
                    *reinterpret_cast<uint2 *>(blk) = uint2{__builtin_amdgcn_perm(v.y, v.x, kEvenBytes),
                                                            __builtin_amdgcn_perm(v.w, v.z, kEvenBytes)};
                    *reinterpret_cast<uint2 *>(blk + 16) = uint2{__builtin_amdgcn_perm(v.y, v.x, kOddBytes),
                                                                 __builtin_amdgcn_perm(v.w, v.z, kOddBytes)};
                    int t = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, 0, false);
                    t = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, t, false);
                    t = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, t, false);
                    t = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, t, false);
                    if constexpr (kXSum)
                        atomicAdd(&xsum[(c * 16) / K], t);
                    csum = t;
                }
            }
            if constexpr (kGXSum) {
                // the GS / 16 chunks of a (token, group) sit on consecutive lanes
                const int gsum = group_sum<GS / 16>(csum);
                if ((tid & (GS / 16 - 1)) == 0 && c < nch)
                    xg[(c * 16) / GS] = gsum;
            }
        }
    }
#pragma unroll
    for (int u = kEarlyUnits; u < kMaxUnitsPerWave; ++u)
        issue(u);
    __syncthreads();
    int xs_fused = 0;
    if constexpr (kXSum && FUSED == 1) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            xs_fused += ipart[w];
        __syncthreads();  // ipart is reused for the partials below
    }

    // 4. Dot products, one unit at a time, for every token.  Each unit's
    //    partial is finished as soon as its own weights have arrived.
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t *xm = sx + m * K;
#pragma unroll
        for (int u = 0; u < kMaxUnitsPerWave; ++u) {
            int r, sg;
            if (!unit_of(u, r, sg))  // wavefront-uniform
                break;
            const int unit = wave + u * kWaves;
            const int64_t n = n0 + r;
            int isum = 0;
            float fsum = 0.f;
#pragma unroll
            for (int i = 0; i < SC; ++i) {
                const int c = lane + 64 * i;
                const bool live = c < SEG && (int64_t)sg * SEG + c < KC;
                const int64_t kc = (int64_t)sg * SEG + (live ? c : 0);  // chunk index within the row
                const uint4 w = wv[u][i];
                int d;
                if constexpr (BITS == 8) {
                    d = dot16(w, *reinterpret_cast<const uint4 *>(xm + kc * 16), 0);
                } else {
                    const uint4 xe = *reinterpret_cast<const uint4 *>(xm + kc * 32);
                    const uint4 xo = *reinterpret_cast<const uint4 *>(xm + kc * 32 + 16);
                    const uint4 lo = {w.x & 0x0F0F0F0Fu, w.y & 0x0F0F0F0Fu, w.z & 0x0F0F0F0Fu,
                                      w.w & 0x0F0F0F0Fu};
                    const uint4 hi = {(w.x >> 4) & 0x0F0F0F0Fu, (w.y >> 4) & 0x0F0F0F0Fu,
                                      (w.z >> 4) & 0x0F0F0F0Fu, (w.w >> 4) & 0x0F0F0F0Fu};
                    d = dot16(hi, xo, dot16(lo, xe, 0));
                }
                d = live ? d : 0;
                if constexpr (GS == 0) {
                    isum += d;
                } else {
                    // the LPG lanes of one group: exact group sum, then scale
                    int gsum = group_sum<LPG>(d);
                    const int64_t g = kc / LPG;
                    if ((lane & (LPG - 1)) == 0 && live && n < N) {
                        if constexpr (kGXSum)
                            gsum -= 8 * xg[m * G + g];
                        if constexpr (OUT == OUT_I32)
                            static_cast<int32_t *>(p.out)[(m * N + n) * G + g] = gsum;
                        else
                            fsum += (float)gsum * swv[u][i];
                    }
                }
            }
            if constexpr (GS == 0) {
                const int t = wave_sum_i32(isum);
                if (lane == 0)
                    ipart[m * 64 + unit] = t;
            } else if constexpr (OUT != OUT_I32) {
                const float t = wave_sum_f32(fsum);
                if (lane == 0)
                    part[m * 64 + unit] = t;
            }
        }
    }
    if constexpr (GS != 0 && OUT == OUT_I32)
        return;
    __syncthreads();

    // 5. One thread per (token, row): combine the row's segments in order.
    if (fin) {
        const int m = tid / R, r = fin_r;
        const int64_t n = n0 + r;
        if constexpr (GS == 0) {
            int32_t total = 0;
            for (int sg = 0; sg < NSEG; ++sg)
                total += ipart[m * 64 + r * NSEG + sg];
            if constexpr (kXSum)
                total -= 8 * (FUSED == 1 ? xs_fused : xsum[m]);
            if constexpr (OUT == OUT_I32) {
                static_cast<int32_t *>(p.out)[m * N + n] = total;
            } else {
                const float st = FUSED == 1 ? s_fused : FUSED == 2 ? stok[m] : p.s_tok[m];
                const float y = (float)total * st * fin_sw;
                static_cast<uint16_t *>(p.out)[m * N + n] = out_bits<OUT>(y);
            }
        } else {
            float tot = 0.f;
            for (int sg = 0; sg < NSEG; ++sg)
                tot += part[m * 64 + r * NSEG + sg];
            const float st = FUSED == 1 ? s_fused : FUSED == 2 ? stok[m] : p.s_tok[m];
            static_cast<uint16_t *>(p.out)[m * N + n] = out_bits<OUT>(st * tot);
        }
    }
}

// Split of the weight rows: NSEG = ceil(chunks / 192) segments of SEG chunks
// (at most 3 per lane, whole groups; the last may be shorter), and as many
// rows per workgroup as fit 5 units per wavefront (40 with 8 wavefronts, 20
// with 4).
void plan(GemvParams &p, int bits, int group_size, int waves)
{
    const int KPC = bits == 8 ? 16 : 32;
    const int64_t KC = p.K / KPC;
    const int64_t lpg = group_size ? group_size / KPC : 1;
    const int64_t nseg = (KC + 191) / 192;
    const int64_t seg = ((KC + nseg - 1) / nseg + lpg - 1) / lpg * lpg;
    p.NSEG = (int)nseg;
    p.SEG = (int)seg;
    p.R = (int)(waves * kMaxUnitsPerWave / nseg);
}

template <int BITS, int GS, int OUT, int FUSED, int XR>
hipError_t launch_xr(const GemvParams &p, hipStream_t stream)
{
    const int64_t blocks = (p.N + p.R - 1) / p.R;
    const size_t lds = (size_t)(FUSED == 1 ? 1 : p.M) * (size_t)p.K;
    // chunk slots per lane: 2 when a segment fits in 128 chunks (no load
    // instructions for a slot no lane uses), else 3
    if (p.SEG <= 128)
        hipLaunchKernelGGL((gemv_kernel<BITS, GS, OUT, FUSED, XR, 2>), dim3((unsigned)blocks),
                           dim3(threads_for(FUSED)), lds, stream, p);
    else
        hipLaunchKernelGGL((gemv_kernel<BITS, GS, OUT, FUSED, XR, kMaxChunksPerLane>), dim3((unsigned)blocks),
                           dim3(threads_for(FUSED)), lds, stream, p);
    return hipGetLastError();
}

template <int BITS, int GS, int OUT, int FUSED>
hipError_t launch_one(GemvParams p, hipStream_t stream)
{
    constexpr int kThreads = threads_for(FUSED);
    plan(p, BITS, GS, kThreads / 64);
    if (p.R < 1 || p.SEG > 64 * kMaxChunksPerLane)
        return hipErrorInvalidValue;  // K too long for the per-lane register budget
    if (BITS == 4 && GS != 0 && (FUSED == 1 ? 1 : p.M) * p.K / (GS ? GS : 1) > kMaxGroupSums)
        return hipErrorInvalidValue;
    if (p.M < 1 || p.M > kMaxM || (FUSED == 1 && p.M != 1))
        return hipErrorInvalidValue;
    const int64_t xchunks = FUSED ? p.M * p.K / 8 : p.M * p.K / 16;
    const int64_t per_thread = (xchunks + kThreads - 1) / kThreads;
    if (per_thread <= 2)
        return launch_xr<BITS, GS, OUT, FUSED, 2>(p, stream);
    if (per_thread <= 5)
        return launch_xr<BITS, GS, OUT, FUSED, 5>(p, stream);
    if (per_thread <= 16)
        return launch_xr<BITS, GS, OUT, FUSED, 16>(p, stream);
    return hipErrorInvalidValue;
}

template <int OUT, int FUSED>
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
    switch (group_size) {
    case 0: return launch_one<4, 0, OUT, FUSED>(p, stream);
    case 64: return launch_one<4, 64, OUT, FUSED>(p, stream);
    case 128: return launch_one<4, 128, OUT, FUSED>(p, stream);
    default: return hipErrorInvalidValue;
    }
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
        return dispatch<OUT_F16, 0>(p, a.bits, a.group_size, stream);
    if (a.out_kind == OUT_BF16)
        return dispatch<OUT_BF16, 0>(p, a.bits, a.group_size, stream);
    return dispatch<OUT_I32, 0>(p, a.bits, a.group_size, stream);
}

hipError_t launch_gemv_fused(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const void *wq,
                             const float *s_w, int64_t N, int bits, int group_size, void *y,
                             int8_t *xq_out, float *s_tok_out, int out_kind, hipStream_t stream)
{
    GemvParams p{};
    p.x = x;
    p.wq = static_cast<const uint8_t *>(wq);
    p.s_w = s_w;
    p.M = M;
    p.N = N;
    p.K = K;
    p.ldx = ldx;
    p.out = y;
    p.xq_out = xq_out;
    p.s_tok_out = s_tok_out;
    // one token of up to 256 * 16 chunks of 8 values: the one-token kernel;
    // a longer one goes to the several-token kernel (512 threads hold it)
    if (M == 1 && K / 8 <= threads_for(1) * 16) {
        if (out_kind == OUT_BF16)
            return dispatch<OUT_BF16, 1>(p, bits, group_size, stream);
        return dispatch<OUT_F16, 1>(p, bits, group_size, stream);
    }
    if (out_kind == OUT_BF16)
        return dispatch<OUT_BF16, 2>(p, bits, group_size, stream);
    return dispatch<OUT_F16, 2>(p, bits, group_size, stream);
}

}  // namespace cider
