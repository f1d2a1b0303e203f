// The pages' decode kernel (Cider README, ossradar.top repo page, "Metal
// Kernel Pipeline", Decode (M = 1): a direct matrix-vector product that
// dequantizes the weights on the fly and does not quantize the activation):
//   y[n] = sum_g s_w[n, g] * sum_{k in g} x[k] * q[n, k]
// with x fp16 [K], int8 or packed int4 weight codes q, per-channel (one
// group of K) or per-group scales, fp32 accumulation, y rounded once to fp16
// or bf16.  (The W8A8 path quantizes the token instead; both are offered.)
//
// One pass over the weight matrix, so the kernel is built around HBM:
//   * x is staged once per workgroup in LDS; a row's weights are split into
//     1, 2, 4 or 8 segments of at most 3 16-byte chunks per lane (16 int8
//     or 32 int4 codes per chunk, adjacent lanes adjacent in memory), one
//     wavefront per segment; the workgroup walks the rows with a grid-wide
//     stride, each wavefront loading its next segment while the current one
//     is reduced;
//   * codes become fp16 exactly by placing the offset-binary code u (int8:
//     q + 128; int4: the nibble, q + 8) in the low mantissa bits of 1024
//     (0x6400 | u is 1024 + u) and subtracting 1024 + offset with a packed
//     fp16 add, then v_dot2_f32_f16 multiplies two codes by two activations
//     and accumulates in fp32;
//   * per group, the lanes holding a group's chunks (consecutive lanes) add
//     their partial sums with DPP exchanges and one of them applies the
//     group's scale; per channel the scale is applied once to the row sum.
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

// The weights stream through once: non-temporal loads.
__device__ __forceinline__ uint4 load_stream(const uint8_t *p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBlocksPerCu = 3;  // workgroups per compute unit (rows beyond: grid-stride)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF,
                                                                 0xF, false));
}

// Sum over aligned groups of L lanes (1, 2, 4 or 8): every lane of a group
// ends with the group's sum.
template <int L>
__device__ __forceinline__ float group_sum_f(float v)
{
    if constexpr (L >= 2)
        v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (L >= 4)
        v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (L >= 8)
        v += dpp_f<0x141>(v);  // row_half_mirror
    return v;
}

__device__ __forceinline__ float wave_sum_f(float v)
{
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);  // row_mirror: each row of 16 now holds its sum
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
}

// Two fp16 codes from the two offset-binary bytes b0 (bits 7:0) and b1
// (bits 23:16) of `t`: halves 1024 + u, minus (1024 + offset).
__device__ __forceinline__ half2_t codes_from_bytes(uint32_t t, _Float16 bias)
{
    const uint32_t h = (t & 0x00FF00FFu) | 0x64006400u;
    return __builtin_bit_cast(half2_t, h) - half2_t{bias, bias};
}

__device__ __forceinline__ float dot2(half2_t a, uint32_t x, float acc)
{
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2_t, x), acc, false);
}

// Dot product of one 16-byte weight chunk with its activations (int8: 16
// fp16 values at xs; int4: 32).
template <int BITS>
__device__ __forceinline__ float chunk_dot(uint4 w, const uint16_t *xs, float acc)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    if constexpr (BITS == 8) {
        const uint4 xa = *reinterpret_cast<const uint4 *>(xs);
        const uint4 xb = *reinterpret_cast<const uint4 *>(xs + 8);
        const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t t = wd[d] ^ 0x80808080u;  // u = q + 128
            // bytes 0, 2 -> codes k, k+2; bytes 1, 3 -> k+1, k+3: pair (k, k+1)
            const uint32_t even = __builtin_amdgcn_perm(0u, t, 0x0c010c00u);  // u1 << 16 | u0
            const uint32_t odd = __builtin_amdgcn_perm(0u, t, 0x0c030c02u);   // u3 << 16 | u2
            acc = dot2(codes_from_bytes(even, (_Float16)1152.0f), xv[2 * d], acc);
            acc = dot2(codes_from_bytes(odd, (_Float16)1152.0f), xv[2 * d + 1], acc);
        }
    } else {
        const uint4 xa = *reinterpret_cast<const uint4 *>(xs);
        const uint4 xb = *reinterpret_cast<const uint4 *>(xs + 8);
        const uint4 xc = *reinterpret_cast<const uint4 *>(xs + 16);
        const uint4 xd = *reinterpret_cast<const uint4 *>(xs + 24);
        const uint32_t xv[16] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w,
                                 xc.x, xc.y, xc.z, xc.w, xd.x, xd.y, xd.z, xd.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            // byte j of the word holds k = 2j (low nibble) and k = 2j + 1 (high)
            const uint32_t lo = wd[d] & 0x0F0F0F0Fu;         // u of k = 0, 2, 4, 6
            const uint32_t hi = (wd[d] >> 4) & 0x0F0F0F0Fu;  // u of k = 1, 3, 5, 7
            const uint32_t p01 = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u);  // u(k1) << 16 | u(k0)
            const uint32_t p23 = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u);
            const uint32_t p45 = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u);
            const uint32_t p67 = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u);
            acc = dot2(codes_from_bytes(p01, (_Float16)1032.0f), xv[4 * d], acc);
            acc = dot2(codes_from_bytes(p23, (_Float16)1032.0f), xv[4 * d + 1], acc);
            acc = dot2(codes_from_bytes(p45, (_Float16)1032.0f), xv[4 * d + 2], acc);
            acc = dot2(codes_from_bytes(p67, (_Float16)1032.0f), xv[4 * d + 3], acc);
        }
    }
    return acc;
}

// A row's K chunks are split into nseg segments (1, 2, 4 or 8) of
// seg_chunks chunks (whole groups), at most SC = 3 per lane; the 8
// wavefronts of a workgroup take 8 / nseg rows at a time, one segment each,
// and walk the rows with a grid-wide stride, loading their next segment while
// the current one is reduced.  Segment sums meet in LDS and are added in
// segment order (results do not depend on timing).
template <int BITS, int GS, int OUT, int SC>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint16_t *__restrict__ x, int64_t K,
                                                          const uint8_t *__restrict__ wq,
                                                          const float *__restrict__ s_w, int64_t N,
                                                          uint16_t *__restrict__ y, int nseg,
                                                          int seg_chunks)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // x [K]
    __shared__ float part[2][kWaves];
    constexpr int KPC = BITS == 8 ? 16 : 32;  // codes per chunk
    constexpr int LPG = GS ? GS / KPC : 1;    // lanes per group
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KC = (int)(K / KPC);
    const int G = GS ? (int)(K / GS) : 1;
    const int64_t wld = BITS == 8 ? K : K / 2;
    const int rpi = kWaves / nseg;  // rows per workgroup and iteration
    const int r_in = wave / nseg, sg = wave % nseg;
    const int c0 = sg * seg_chunks, c1 = min(c0 + seg_chunks, KC);
    const int64_t stride = (int64_t)gridDim.x * rpi;

    // A segment's weight chunks and the scales that go with them (per group:
    // each chunk's group scale; per channel: the row's scale), so that no
    // scale load waits behind the dot products.
    auto load_seg = [&](uint4 (&w)[SC], float (&sc)[SC], int64_t r) {
        const int64_t rr = min(r, N - 1);  // past the end: a valid row, unused
        const uint8_t *row = wq + rr * wld;
#pragma unroll
        for (int j = 0; j < SC; ++j) {
            const int c = min(c0 + lane + 64 * j, KC - 1);  // past the segment: masked below
            w[j] = load_stream(row + (int64_t)c * 16);
            sc[j] = GS ? s_w[rr * G + c / LPG] : (j == 0 ? s_w[rr] : 0.f);
        }
    };
    int64_t base = (int64_t)blockIdx.x * rpi;
    uint4 cur[SC];
    float csc[SC];
    load_seg(cur, csc, base + r_in);
    for (int64_t i = threadIdx.x; i < K / 8; i += kThreads)
        *reinterpret_cast<uint4 *>(xs + i * 8) = *reinterpret_cast<const uint4 *>(x + i * 8);
    __syncthreads();

    for (int it = 0; base < N; base += stride, ++it) {  // workgroup-uniform
        const int64_t row = base + r_in;
        uint4 nxt[SC];
        float nsc[SC];
        load_seg(nxt, nsc, base + stride + r_in);
        float total = 0.f;
#pragma unroll
        for (int j = 0; j < SC; ++j) {
            const int c = c0 + lane + 64 * j;
            const bool live = c < c1 && row < N;
            float p = chunk_dot<BITS>(cur[j], xs + (int64_t)min(c, KC - 1) * KPC, 0.f);
            p = live ? p : 0.f;
            if constexpr (GS == 0) {
                total += p;
            } else {
                const float gsum = group_sum_f<LPG>(p);
                if ((lane & (LPG - 1)) == 0 && live)
                    total += gsum * csc[j];
            }
        }
        const float t = wave_sum_f(total);
        if (lane == 0)
            part[it & 1][wave] = t;
        __syncthreads();  // part[it & 1] is rewritten two iterations later, after another barrier
        if (sg == 0 && lane == 0 && row < N) {
            float r = part[it & 1][wave];
            for (int q = 1; q < nseg; ++q)
                r += part[it & 1][wave + q];
            if constexpr (GS == 0)
                r *= csc[0];
            y[row] = out_bits<OUT>(r);
        }
#pragma unroll
        for (int j = 0; j < SC; ++j) {
            cur[j] = nxt[j];
            csc[j] = nsc[j];
        }
    }
}

int compute_units()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int BITS, int GS, int OUT, int SC>
hipError_t launch_sc(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                     void *y, int nseg, int seg_chunks, hipStream_t stream)
{
    const int rpi = kWaves / nseg;
    const int64_t blocks = std::min<int64_t>((N + rpi - 1) / rpi, (int64_t)compute_units() * kBlocksPerCu);
    hipLaunchKernelGGL((decode_kernel<BITS, GS, OUT, SC>), dim3((unsigned)blocks), dim3(kThreads),
                       (size_t)K * 2, stream, x, K, static_cast<const uint8_t *>(wq), s_w, N,
                       static_cast<uint16_t *>(y), nseg, seg_chunks);
    return hipGetLastError();
}

// Segments: the fewest of 1, 2, 4, 8 that leave at most 3 chunks per lane,
// each a whole number of groups.
template <int BITS, int GS, int OUT>
hipError_t launch_mode(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                       void *y, hipStream_t stream)
{
    constexpr int KPC = BITS == 8 ? 16 : 32;
    constexpr int LPG = GS ? GS / KPC : 1;
    const int64_t chunks = K / KPC;
    int nseg = 1;
    while (nseg < kWaves && (chunks + nseg - 1) / nseg > 192)
        nseg *= 2;
    const int64_t seg = ((chunks + nseg - 1) / nseg + LPG - 1) / LPG * LPG;
    const int64_t sc = (seg + 63) / 64;
    if (sc <= 1)
        return launch_sc<BITS, GS, OUT, 1>(x, K, wq, s_w, N, y, nseg, (int)seg, stream);
    if (sc <= 2)
        return launch_sc<BITS, GS, OUT, 2>(x, K, wq, s_w, N, y, nseg, (int)seg, stream);
    if (sc <= 3)
        return launch_sc<BITS, GS, OUT, 3>(x, K, wq, s_w, N, y, nseg, (int)seg, stream);
    return hipErrorInvalidValue;
}

template <int OUT>
hipError_t launch_out(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                      int bits, int group_size, void *y, hipStream_t stream)
{
    if (bits == 8) {
        switch (group_size) {
        case 0: return launch_mode<8, 0, OUT>(x, K, wq, s_w, N, y, stream);
        case 64: return launch_mode<8, 64, OUT>(x, K, wq, s_w, N, y, stream);
        case 128: return launch_mode<8, 128, OUT>(x, K, wq, s_w, N, y, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (group_size) {
    case 0: return launch_mode<4, 0, OUT>(x, K, wq, s_w, N, y, stream);
    case 64: return launch_mode<4, 64, OUT>(x, K, wq, s_w, N, y, stream);
    case 128: return launch_mode<4, 128, OUT>(x, K, wq, s_w, N, y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                         int bits, int group_size, int out_kind, void *y, hipStream_t stream)
{
    if (N == 0)
        return hipSuccess;
    return out_kind == OUT_BF16 ? launch_out<OUT_BF16>(x, K, wq, s_w, N, bits, group_size, y, stream)
                                : launch_out<OUT_F16>(x, K, wq, s_w, N, bits, group_size, y, stream);
}

}  // namespace cider
