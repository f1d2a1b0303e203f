// Matrix-core product for few tokens (M <= 256) with per-group scaling
// (Cider README, ossradar.top repo page, "Quantization" table: INT32
// accumulation, C_fp16 = C_int32 * s_act * s_weight; "W8A8 Quantization
// Granularity": one scale per group of 64 or 128; "TensorOps matmul2d": tile
// shape chosen by M, small tiles for small M).  The kernel is written for
// every mode; per channel the large-M kernel's small tile is faster at these
// M (measured), so only per-group products are dispatched here.
//
// With few tokens the weight matrix is read once and the work per weight
// byte is small, so the product is bound by how fast the weights stream in.
// The large-M kernel walks K serially inside a workgroup; here each
// workgroup owns a small TN-channel x TM-token tile and its 8 wavefronts
// split K among themselves:
//   * a wavefront takes every 8th K unit of 128 values and loads
//     its MFMA fragments straight from global memory into registers
//     (range-checked buffer loads, out-of-range rows read as zeros), one or
//     two units ahead of the MFMAs;
//   * v_mfma_i32_16x16x64_i8: its operand layout (16 rows, four 16-byte
//     chunks of 64 values) makes every fragment load read 64 contiguous bytes
//     per row, where the 32 x 32 x 32 layout would read 32 bytes from each of
//     32 rows (twice the cache accesses per byte; the matrix cores are far
//     from busy here, so the slower instruction costs nothing).  Per channel
//     the weight fragment is operand A (a lane's outputs are 4 consecutive
//     channels of a token); per group the roles swap (a lane's outputs are 4
//     tokens of one channel), each group's int32 sums scaled into fp32 once
//     the group ends;
//   * int4 weights are widened in registers (q = u - 8) right before use;
//   * the wavefronts' partial tiles meet in LDS -- int32 sums through LDS
//     integer atomics (exact), per-group fp32 sums added in wavefront order --
//     so results do not depend on timing; then dequantized and stored as
//     contiguous fp16 rows.
#include "cider_kernels.h"

namespace cider {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, range-checked dwords
constexpr uint32_t kDead = 0x80000000u;  // past every operand: loads return zero

__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// 8 packed nibbles (low nibble = even k) -> int8 codes q = u - 8, k order kept.
__device__ __forceinline__ void widen8(uint32_t v, uint32_t &d0, uint32_t &d1)
{
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // k0 k1 k2 k3
    const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // k4 k5 k6 k7
    d0 = (a + 0x78787878u) ^ 0x80808080u;
    d1 = (b + 0x78787878u) ^ 0x80808080u;
}

// TN channels x TM tokens per workgroup; a K unit is 128 values deep: two
// 64-deep steps of v_mfma_i32_16x16x64_i8 (per group a unit holds 128 / GS
// whole groups).  Fragment loads follow that instruction's operand layout --
// lane l takes row l % 16 and the 16-byte chunk l / 16 of the step -- so one
// load reads 64 contiguous bytes of each of 16 rows (int4 weights: 32).
template <int TN, int TM, int BITS, int GS, int OUT>
__global__ __launch_bounds__(kThreads) void skinny_kernel(ProductArgs args, int tiles_n)
{
    constexpr int FN = TN / 16, FM = TM / 16;
    constexpr bool PG = GS != 0;
    constexpr int U = 128;
    constexpr int STEPS = U / 64;
    constexpr int GPU = PG ? U / GS : 1;          // groups per unit
    constexpr int SPG = PG ? GS / 64 : STEPS;     // steps per group
    constexpr int WB = BITS == 8 ? 16 : 8;        // weight fragment bytes per lane per step
    constexpr int WSTEP = BITS == 8 ? 64 : 32;    // weight row bytes per step
    // units loaded ahead of the MFMAs: 2, or 1 when a unit's fragments are large
    constexpr int kAhead = STEPS * (FN + FM) * 4 > 48 ? 1 : 2;
    // Partial tiles, [token][channel] with rows padded by one word.  Per
    // channel one int32 tile that every wavefront adds into with LDS integer
    // atomics (exact, so the order does not matter); per group one fp32 tile
    // per wavefront, added in wavefront order afterwards.
    constexpr int TS = TN + 1;
    constexpr int NPART = PG ? kWaves : 1;
    __shared__ int32_t part[NPART * TM * TS];
    __shared__ float s_st[TM], s_sw[TN];  // dequant scales of the tile

    const int64_t M = args.M, N = args.N, K = args.K;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int frow = lane & 15, fq = lane >> 4;  // fragment row, 16-byte chunk
    const int64_t wld = BITS == 8 ? K : K / 2;
    const int G = PG ? (int)(K / GS) : 1;

    // Zero the int32 tile.  The tile's scales go into registers now
    // (branch-free loads whose latency hides under the main loop) and into
    // LDS just before the reduction's barrier: stored to LDS here, every
    // wavefront would wait for them before issuing its first weight load.
    if constexpr (!PG)
        for (int o = threadIdx.x; o < TM * TS; o += kThreads)
            part[o] = 0;
    constexpr int NSV = PG ? TM : TM + TN;  // per group, channel scales come per unit
    constexpr int NSC = OUT != OUT_I32 ? (NSV + kThreads - 1) / kThreads : 0;
    float scv[NSC > 0 ? NSC : 1];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int o = (int)threadIdx.x + i * kThreads;
        const float *src = o < TM ? args.s_tok + min(m0 + o, M - 1)
                                  : args.s_w + min(n0 + min(o - TM, TN - 1), N - 1);
        scv[i] = *src;
    }
    __syncthreads();

    const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)args.xq, (short)0, (int)(M * K), kRsrcWord3);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)args.wq, (short)0, (int)(N * wld), kRsrcWord3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)args.s_w, (short)0,
                                                      (OUT != OUT_I32 && PG) ? (int)(N * G * 4) : 0,
                                                      kRsrcWord3);

    // This wavefront's units: wave, wave + 8, ... (at any moment the 8
    // wavefronts read adjacent 128-byte pieces of the same rows).
    const int KU = (int)((K + U - 1) / U);  // K % 64 == 0: the last unit may hold one step
    const int nu = KU > wave ? (KU - wave + kWaves - 1) / kWaves : 0;  // units of this wavefront

    // Row offsets of this lane's fragment rows (rows past the operand read 0).
    uint32_t xrow[FM], wrow[FN];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + j * 16 + frow;
        xrow[j] = m < M ? (uint32_t)(m * K) + fq * 16 : kDead;
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int64_t n = n0 + i * 16 + frow;
        wrow[i] = n < N ? (uint32_t)(n * wld) + fq * WB : kDead;
    }

    struct Unit {
        i32x4 x[STEPS][FM];
        i32x4 w[BITS == 8 ? STEPS : 1][BITS == 8 ? FN : 1];   // int8 codes
        uint2 wp[BITS == 4 ? STEPS : 1][BITS == 4 ? FN : 1];  // packed int4
        float sw[PG ? GPU : 1][PG ? FN : 1];
    };
    auto load_unit = [&](Unit &t, int ui) {  // ui: this wavefront's ui-th unit
        const bool live = ui < nu;
        const int u = wave + ui * kWaves;
        const uint32_t kx = (uint32_t)u * U;                  // byte offset in an X row
        const uint32_t kw = BITS == 8 ? kx : kx / 2;          // byte offset in a W row
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const bool ls = live && kx + s * 64 < (uint32_t)K;  // steps past K read zeros
#pragma unroll
            for (int j = 0; j < FM; ++j)
                t.x[s][j] = load16(rx, ls ? xrow[j] + kx + s * 64 : kDead);
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                if constexpr (BITS == 8)
                    t.w[s][i] = load16(rw, ls ? wrow[i] + kw + s * WSTEP : kDead);
                else
                    t.wp[s][i] = load8(rw, ls ? wrow[i] + kw + s * WSTEP : kDead);
            }
        }
        if constexpr (PG && OUT != OUT_I32) {
#pragma unroll
            for (int q = 0; q < GPU; ++q)
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int64_t n = n0 + i * 16 + frow;
                    const int64_t g = (int64_t)u * GPU + q;
                    const uint32_t off = (uint32_t)(n * G + g) * 4u;
                    t.sw[q][i] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rs, live && n < N && g < G ? off : kDead, 0, 0));
                }
        }
    };

    i32x4 acc[FN][FM];
    float facc[PG ? FN : 1][PG ? FM : 1][PG ? 4 : 1];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            acc[i][j] = i32x4{};
            if constexpr (PG)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    facc[i][j][e] = 0.f;
        }

    Unit ring[kAhead + 1];
#pragma unroll
    for (int p = 0; p < kAhead; ++p)
        load_unit(ring[p], p);
    for (int ub = 0; ub < nu; ub += kAhead + 1) {
#pragma unroll
        for (int r = 0; r < kAhead + 1; ++r) {
            const int ui = ub + r;
            if (ui >= nu)  // wavefront-uniform
                break;
            const int uu = wave + ui * kWaves;  // the unit's index along K
            load_unit(ring[(r + kAhead) % (kAhead + 1)], ui + kAhead);
            Unit &t = ring[r];
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    i32x4 wf;
                    if constexpr (BITS == 8) {
                        wf = t.w[s][i];
                    } else {
                        uint32_t d0, d1, d2, d3;
                        widen8(t.wp[s][i].x, d0, d1);
                        widen8(t.wp[s][i].y, d2, d3);
                        wf = i32x4{(int)d0, (int)d1, (int)d2, (int)d3};
                    }
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        if constexpr (!PG)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, t.x[s][j], acc[i][j], 0, 0, 0);
                        else if (s % SPG == 0)  // a group opens: start from zero
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(t.x[s][j], wf, i32x4{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(t.x[s][j], wf, acc[i][j], 0, 0, 0);
                    }
                }
                if constexpr (PG) {
                    if (s % SPG == SPG - 1) {  // a group closes: scale it, or store it (int32 hook)
                        const int q = s / SPG;
                        const int64_t g = (int64_t)uu * GPU + q;
#pragma unroll
                        for (int i = 0; i < FN; ++i) {
                            const int64_t n = n0 + i * 16 + frow;
#pragma unroll
                            for (int j = 0; j < FM; ++j)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    if constexpr (OUT != OUT_I32) {
                                        facc[i][j][e] += (float)acc[i][j][e] * t.sw[q][i];
                                    } else {
                                        const int64_t m = m0 + j * 16 + fq * 4 + e;
                                        if (m < M && n < N && g < G)
                                            static_cast<int32_t *>(args.out)[(m * N + n) * G + g] = acc[i][j][e];
                                    }
                                }
                        }
                    }
                }
            }
        }
    }
    if constexpr (PG && OUT == OUT_I32)
        return;

    if constexpr (OUT != OUT_I32) {
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int o = (int)threadIdx.x + i * kThreads;
            if (o < TM)
                s_st[o] = scv[i];
            else if (o < NSV)
                s_sw[o - TM] = scv[i];
        }
    }

    // Partial tiles to LDS.  Block (i, j) gives the lane: per channel, token
    // 16j + lane%16 and channels 16i + 4*(lane/16) + e; per group, channel
    // 16i + lane%16 and tokens 16j + 4*(lane/16) + e.
    int32_t *mine = part + (PG ? wave : 0) * TM * TS;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (!PG) {
                    const int t = j * 16 + frow, c = i * 16 + fq * 4 + e;
                    atomicAdd(&mine[t * TS + c], acc[i][j][e]);
                } else {
                    const int t = j * 16 + fq * 4 + e, c = i * 16 + frow;
                    mine[t * TS + c] = __builtin_bit_cast(int32_t, facc[i][j][e]);
                }
            }
    __syncthreads();

    // Sum the wavefronts' partials in order, dequantize, store.
    for (int o = threadIdx.x; o < TM * TN; o += kThreads) {
        const int t = o / TN, c = o % TN;
        const int64_t m = m0 + t, n = n0 + c;
        if (m >= M || n >= N)
            continue;
        if constexpr (!PG) {
            const int32_t total = part[t * TS + c];
            if constexpr (OUT == OUT_I32) {
                static_cast<int32_t *>(args.out)[m * N + n] = total;
            } else {
                const float y = (float)total * s_st[t] * s_sw[c];
                static_cast<uint16_t *>(args.out)[m * N + n] = out_bits<OUT>(y);
            }
        } else {
            float total = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                total += __builtin_bit_cast(float, part[w * TM * TS + t * TS + c]);
            const float y = s_st[t] * total;
            static_cast<uint16_t *>(args.out)[m * N + n] = out_bits<OUT>(y);
        }
    }
}

template <int TN, int TM, int BITS, int GS, int OUT>
hipError_t launch_tile(const ProductArgs &a, hipStream_t stream)
{
    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    hipLaunchKernelGGL((skinny_kernel<TN, TM, BITS, GS, OUT>), dim3(tiles_n * tiles_m), dim3(kThreads), 0,
                       stream, a, tiles_n);
    return hipGetLastError();
}

// The largest tile that still gives at least 256 workgroups (else the
// smallest): 64 x 64, 64 x 32, 32 x 64, 32 x 32 (channels x tokens).  Per
// group always 32 x 32 (the fp32 sums and group scales need the registers).
template <int BITS, int GS, int OUT>
hipError_t launch_mode(const ProductArgs &a, hipStream_t stream)
{
    auto tiles = [&](int tn, int tm) { return ((a.N + tn - 1) / tn) * ((a.M + tm - 1) / tm); };
    if constexpr (GS == 0) {
        if (a.M > 32 && tiles(64, 64) >= 256)
            return launch_tile<64, 64, BITS, GS, OUT>(a, stream);
        if (tiles(64, 32) >= 256)
            return launch_tile<64, 32, BITS, GS, OUT>(a, stream);
        if (a.M > 32 && tiles(32, 64) >= 256)
            return launch_tile<32, 64, BITS, GS, OUT>(a, stream);
    }
    return launch_tile<32, 32, BITS, GS, OUT>(a, stream);
}

// Per-group products only: per channel, the large-M kernel's 64 x 128 tile
// with its deep copy ring is faster at these M (measured).
template <int BITS, int OUT>
hipError_t launch_group(const ProductArgs &a, hipStream_t stream)
{
    switch (a.group_size) {
    case 64: return launch_mode<BITS, 64, OUT>(a, stream);
    case 128: return launch_mode<BITS, 128, OUT>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int OUT>
hipError_t launch_out(const ProductArgs &a, hipStream_t stream)
{
    return a.bits == 8 ? launch_group<8, OUT>(a, stream) : launch_group<4, OUT>(a, stream);
}

}  // namespace

hipError_t launch_gemm_skinny(const ProductArgs &a, hipStream_t stream)
{
    switch (a.out_kind) {
    case OUT_F16: return launch_out<OUT_F16>(a, stream);
    case OUT_BF16: return launch_out<OUT_BF16>(a, stream);
    default: return launch_out<OUT_I32>(a, stream);
    }
}

}  // namespace cider
