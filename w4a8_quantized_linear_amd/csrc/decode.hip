// The pages' decode kernel (Cider README, ossradar.top repo page, "Metal
// Kernel Pipeline", Decode (M = 1): a direct matrix-vector product that
// dequantizes the weights on the fly and does not quantize the activation):
//   y[n] = sum_g s_w[n, g] * sum_{k in g} x[k] * q[n, k]
// with x fp16 [K], int8 or packed int4 weight codes q, per-channel (one
// group of K) or per-group scales, fp32 accumulation, y rounded once to fp16
// or bf16.  (The W8A8 path quantizes the token instead; both are offered.)
//
// One pass over the weight matrix, so the kernel is built around HBM:
//   * a workgroup of 4 wavefronts owns R consecutive rows, split into
//     K-segments of at most 3 16-byte chunks per lane (16 int8 or 32 int4
//     codes per chunk, adjacent lanes adjacent in memory); its (row, segment)
//     units are dealt 5 to a wavefront, and every unit's loads are issued
//     before any arithmetic, up to 15 per lane in flight (two units' worth
//     before x is written to LDS, the rest after);
//   * x is loaded once per workgroup into LDS while the weights are in flight,
//     laid out so that a wavefront's 16-byte reads hit consecutive slots (no
//     bank conflicts); for int4 each 8 values are reordered even k then odd k;
//   * codes become fp16 exactly: one v_perm_b32 pairs two offset-binary codes
//     u (int8: q + 128; int4: the low nibble, q + 8, or the high nibble kept
//     in place, 16 (q + 8)) each under the byte 0x64, giving halves 1024 + u;
//     a packed fp16 subtraction of 1024 + offset leaves the signed codes, and
//     v_dot2_f32_f16 multiplies two codes by two activations and accumulates
//     in fp32 (the high-nibble sum is scaled by 1/16 at the end, exactly);
//   * per group, the lanes holding a group's chunks (consecutive lanes) add
//     their partial sums with DPP exchanges and one of them applies the
//     group's scale; per channel the scale is applied once to the row sum.
#include "cider_kernels.h"
#include "quant_common.h"

namespace cider {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnits = 5;   // (row, segment) units per wavefront
constexpr int kChunks = 3;  // 16-byte chunks per lane and unit, at most
constexpr int kEarly = 2;   // units whose loads go out before x is written to LDS
static_assert(kWaves * kUnits <= kThreads, "one finishing thread per row");

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

// Two fp16 codes from a 32-bit word whose bytes 1 and 3 are 0x64 and whose
// bytes 0 and 2 are offset-binary codes u: the halves are 1024 + u, minus
// `bias` (1024 + the offset) gives the signed codes exactly.
__device__ __forceinline__ half2_t codes_of(uint32_t h, _Float16 bias)
{
    return __builtin_bit_cast(half2_t, h) - half2_t{bias, bias};
}

__device__ __forceinline__ float dot2(half2_t a, uint32_t x, float acc)
{
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2_t, x), acc, false);
}

// v_perm_b32 selectors over {0x64646464 : t}: bytes 0, 1 (or 2, 3) of t,
// each followed by 0x64.
constexpr uint32_t kHigh = 0x64646464u;
constexpr uint32_t kPair01 = 0x04010400u;
constexpr uint32_t kPair23 = 0x04030402u;

// x sits in LDS as 16-byte pieces, piece p of chunk c at 16-byte slot
// p * KC + c, so that the 64 lanes of a wavefront, which hold 64 consecutive
// chunks, read 64 consecutive slots.  int8: a chunk's 16 values are 2
// pieces in natural order.  int4: 4 pieces of 8 values, each ordered
// x0 x2 x4 x6 x1 x3 x5 x7 to match the low (even k) and high (odd k)
// nibbles of one weight word.
template <int BITS>
__device__ __forceinline__ int x_slot(int j, int KC)  // slot of the j-th 8 values
{
    constexpr int P = BITS == 8 ? 2 : 4;
    return (j % P) * KC + j / P;
}

template <int BITS>
__device__ __forceinline__ uint4 x_piece(uint4 v)
{
    if constexpr (BITS == 8)
        return v;
    return uint4{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                 __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
}

// Dot product of weight chunk c (16 bytes) with its activations.
template <int BITS>
__device__ __forceinline__ float chunk_dot(uint4 w, const uint4 *xs, int KC, int c)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    if constexpr (BITS == 8) {
        const uint4 xa = xs[c], xb = xs[KC + c];
        const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t t = wd[d] ^ 0x80808080u;  // u = q + 128, codes k .. k + 3
            acc = dot2(codes_of(__builtin_amdgcn_perm(kHigh, t, kPair01), (_Float16)1152.0f), xv[2 * d], acc);
            acc = dot2(codes_of(__builtin_amdgcn_perm(kHigh, t, kPair23), (_Float16)1152.0f), xv[2 * d + 1], acc);
        }
        return acc;
    } else {
        // Low nibbles: u of k = 0, 2, 4, 6 of the word.  High nibbles, kept
        // in place: 16 u of k = 1, 3, 5, 7, so their codes are 16 q (exact)
        // and their sum is scaled by 1/16 (exact) at the end.
        float even = 0.f, odd = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4 xp = xs[d * KC + c];
            const uint32_t lo = wd[d] & 0x0F0F0F0Fu, hi = wd[d] & 0xF0F0F0F0u;
            even = dot2(codes_of(__builtin_amdgcn_perm(kHigh, lo, kPair01), (_Float16)1032.0f), xp.x, even);
            even = dot2(codes_of(__builtin_amdgcn_perm(kHigh, lo, kPair23), (_Float16)1032.0f), xp.y, even);
            odd = dot2(codes_of(__builtin_amdgcn_perm(kHigh, hi, kPair01), (_Float16)1152.0f), xp.z, odd);
            odd = dot2(codes_of(__builtin_amdgcn_perm(kHigh, hi, kPair23), (_Float16)1152.0f), xp.w, odd);
        }
        return even + odd * 0.0625f;
    }
}

// Work split: a row's K chunks form NSEG = ceil(chunks / 192) segments of
// SEG chunks (whole groups, at most 3 per lane); a workgroup owns R
// consecutive rows, and its R * NSEG (row, segment) units are dealt
// round-robin to its wavefronts, kUnits each.
struct DecodeParams {
    const uint16_t *x;  // fp16 [K]
    const uint8_t *wq;  // int8 [N, K] or packed int4 [N, K / 2]
    const float *s_w;   // [N] or [N, K / GS]
    uint16_t *y;        // [N]
    int64_t N, K;
    int R, NSEG, SEG;
};

constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor: raw dwords, range-checked
constexpr uint32_t kDead = 0x80000000u;  // past every buffer's range: the load returns zero

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The weights stream through once: non-temporal loads (cache policy nt).
__device__ __forceinline__ uint4 load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Each workgroup runs once.  The memory counter retires loads in order, so
// the loads go out in the order they are needed: the activation chunks (XR
// per thread), the first kEarly units' weight chunks (and per group their
// scales) and the row scale of the output this thread finishes; the
// activation is written to LDS as soon as its own loads are back, then the
// remaining units' loads go out, and each unit's dot products start as soon
// as that unit's weights are in.  Unit sums meet in LDS
// and a row's segments are added in segment order (results do not depend on
// timing).  Rows and chunks past the end read zeros through the buffer
// descriptors' range checks and are never stored.
template <int BITS, int GS, int OUT, int XR, int SC>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // x [K]
    __shared__ float part[kWaves * kUnits];                         // [unit] sums
    constexpr int KPC = BITS == 8 ? 16 : 32;  // codes per chunk
    constexpr int LPG = GS ? GS / KPC : 1;    // lanes per group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = p.N, K = p.K;
    const int R = p.R, NSEG = p.NSEG, SEG = p.SEG;
    const int units = R * NSEG;
    const int KC = (int)(K / KPC);
    const int G = GS ? (int)(K / GS) : 1;
    const uint32_t wld = (uint32_t)(BITS == 8 ? K : K / 2);
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int rows = (int)min<int64_t>(R, N - n0);  // rows of this workgroup that exist

    const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, (short)0, (int)(K * 2), kRsrcWord3);
    uint4 xr[XR];
#pragma unroll
    for (int j = 0; j < XR; ++j)
        xr[j] = load16(rx, (uint32_t)(tid + j * kThreads) * 16u);

    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)(p.wq + n0 * wld), (short)0,
                                                      (int)(rows * wld), kRsrcWord3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.s_w + n0 * G), (short)0,
                                                      rows * G * 4, kRsrcWord3);
    uint4 wv[kUnits][SC];
    float swv[GS ? kUnits : 1][GS ? SC : 1];
    auto issue = [&](int u) __attribute__((always_inline)) {
        const int unit = wave + u * kWaves;
        const int r = unit / NSEG, sg = unit % NSEG;
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int c = lane + 64 * i, kc = sg * SEG + c;
            const bool live = unit < units && c < SEG && kc < KC;
            wv[u][i] = load16_stream(rw, live ? (uint32_t)r * wld + (uint32_t)kc * 16u : kDead);
            if constexpr (GS != 0)
                swv[u][i] = load_f32(rs, live ? (uint32_t)(r * G + kc / LPG) * 4u : kDead);
        }
    };
#pragma unroll
    for (int u = 0; u < kEarly; ++u)
        issue(u);
    float fin_sw = 0.f;
    if constexpr (GS == 0)
        fin_sw = load_f32(rs, tid < rows ? (uint32_t)tid * 4u : kDead);

#pragma unroll
    for (int j = 0; j < XR; ++j) {
        const int c = tid + j * kThreads;
        if (c < (int)(K / 8))
            reinterpret_cast<uint4 *>(xs)[x_slot<BITS>(c, KC)] = x_piece<BITS>(xr[j]);
    }
#pragma unroll
    for (int u = kEarly; u < kUnits; ++u)
        issue(u);
    __syncthreads();

#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const int unit = wave + u * kWaves;
        if (unit >= units)  // wavefront-uniform
            break;
        const int sg = unit % NSEG;
        float total = 0.f;
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            if (64 * i >= SEG)  // wavefront-uniform: no lane holds a chunk here
                break;
            const int c = lane + 64 * i, kc = sg * SEG + c;
            const bool live = c < SEG && kc < KC;
            float d = chunk_dot<BITS>(wv[u][i], reinterpret_cast<const uint4 *>(xs), KC, live ? kc : 0);
            d = live ? d : 0.f;
            if constexpr (GS == 0) {
                total += d;
            } else {
                const float gsum = group_sum_f<LPG>(d);  // the group's LPG lanes are all live or all not
                if ((lane & (LPG - 1)) == 0 && live)
                    total += gsum * swv[u][i];
            }
        }
        const float t = wave_sum_f(total);
        if (lane == 0)
            part[unit] = t;
    }
    __syncthreads();

    if (tid < rows) {
        float r = 0.f;
        for (int sg = 0; sg < NSEG; ++sg)
            r += part[tid * NSEG + sg];
        if constexpr (GS == 0)
            r *= fin_sw;
        p.y[n0 + tid] = out_bits<OUT>(r);
    }
}

template <int BITS, int GS, int OUT, int XR>
hipError_t launch_xr(const DecodeParams &p, hipStream_t stream)
{
    const int64_t blocks = (p.N + p.R - 1) / p.R;
    // chunk slots per lane: 2 when a segment fits in 128 chunks (no load
    // instructions for a slot no lane uses), else 3
    if (p.SEG <= 128)
        hipLaunchKernelGGL((decode_kernel<BITS, GS, OUT, XR, 2>), dim3((unsigned)blocks), dim3(kThreads),
                           (size_t)p.K * 2, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<BITS, GS, OUT, XR, kChunks>), dim3((unsigned)blocks), dim3(kThreads),
                           (size_t)p.K * 2, stream, p);
    return hipGetLastError();
}

template <int BITS, int GS, int OUT>
hipError_t launch_mode(const uint16_t *x, int64_t K, const void *wq, const float *s_w, int64_t N,
                       void *y, hipStream_t stream)
{
    constexpr int KPC = BITS == 8 ? 16 : 32;
    constexpr int LPG = GS ? GS / KPC : 1;
    const int64_t chunks = K / KPC;
    const int64_t nseg = (chunks + 64 * kChunks - 1) / (64 * kChunks);
    const int64_t seg = ((chunks + nseg - 1) / nseg + LPG - 1) / LPG * LPG;
    DecodeParams p{x, static_cast<const uint8_t *>(wq), s_w, static_cast<uint16_t *>(y), N, K,
                   (int)(kWaves * kUnits / nseg), (int)nseg, (int)seg};
    // one 16-byte activation chunk (8 values) per thread and XR
    const int64_t xr = (K / 8 + kThreads - 1) / kThreads;
    if (p.R < 1 || seg > 64 * kChunks)
        return hipErrorInvalidValue;  // K too long for the per-lane register budget
    if (xr <= 1)
        return launch_xr<BITS, GS, OUT, 1>(p, stream);
    if (xr <= 2)
        return launch_xr<BITS, GS, OUT, 2>(p, stream);
    if (xr <= 4)
        return launch_xr<BITS, GS, OUT, 4>(p, stream);
    if (xr <= 8)
        return launch_xr<BITS, GS, OUT, 8>(p, stream);
    if (xr <= 16)
        return launch_xr<BITS, GS, OUT, 16>(p, stream);
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
