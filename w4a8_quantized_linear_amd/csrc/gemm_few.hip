// Matrix-core product for a few tokens (up to 32 per tile; per group without
// a split workspace, tiles repeated over up to 256 tokens), every mode: the
// int32 sums of int8 x int8 (or widened int4) products, dequantized in the
// epilogue (Cider README, ossradar.top repo page, "Quantization" table:
// INT32 accumulation, C_fp16 = C_int32 * s_act * s_weight; "W8A8
// Quantization Granularity": one scale per channel or per group of 64 / 128;
// "TensorOps matmul2d": small tiles for small M).
//
// With this few tokens the weight matrix is read once and each weight byte
// takes part in at most 32 multiply-adds, so the product runs at the rate the
// weights stream in.  The kernel is laid out for that stream:
//   * a wavefront owns RBW blocks of 16 weight rows and every KS-th K unit
//     (one 128-byte line of each row: 128 int8 or 256 int4 values); the KS
//     wavefronts that share rows read adjacent lines of them at any moment;
//   * weights arrive as whole 128-byte lines -- eight rows per load,
//     adjacent lanes on adjacent 16 bytes -- with the non-temporal hint, R
//     units ahead of the matrix cores and with no barrier on the way; a load
//     straight into the matrix-core operand layout would read 64 bytes from
//     each of 16 rows instead, which streams ~20 % slower (measured);
//   * each wavefront turns its lines into operand fragments through a
//     private 2 KB LDS slot per 16-row block (write in load order, read in
//     fragment order, XOR-swizzled so that neither side has bank conflicts
//     on 64 banks); token lines take the same route;
//   * v_mfma_i32_16x16x64_i8.  Per channel the weights are operand A (a
//     lane's four outputs are four channels of one token); per group the
//     roles swap (four tokens of one channel, one group scale per lane and
//     block) and each group's int32 sums are scaled into fp32 as it closes;
//   * int4 weights are widened to q = u - 8 right after the fragment read;
//   * the KS partial tiles meet in LDS and are added in K-split order (so
//     results do not depend on timing), dequantized and stored two outputs
//     per 4-byte store.
#include "cider_kernels.h"

namespace cider {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, range-checked dwords
constexpr uint32_t kDead = 0x80000000u;  // past every operand: loads return zero
constexpr int kSlot = 2048;              // one 16-row x 128-byte block

template <int AUX>
__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
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

// Byte offset of 16-byte chunk c (0..7) of row r (0..15) in a slot: rows of
// 128 bytes, chunk index XOR (r / 2) % 8.  A 16-lane pass of the fragment
// read (rows 0..15, one chunk) and of the line write (two rows, chunks
// 0..7) each cover 16 distinct 16-byte bank groups of a 256-byte bank row.
__device__ __forceinline__ uint32_t slot_off(int r, int c)
{
    return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

// BITS 8 / 4; GS 0 (per channel) / 64 / 128; OUT fp16, bf16 or int32 (int32
// per channel only); MT tokens per tile (16 / 32); RBW 16-row blocks per
// wavefront; RG row groups and KS K-splits per workgroup (RG * KS
// wavefronts, NB = 16 * RBW * RG channels); R units in flight per wavefront.
template <int BITS, int GS, int OUT, int MT, int RBW, int RG, int KS, int R>
__global__ __launch_bounds__(64 * RG * KS) void few_kernel(ProductArgs args, int tiles_n)
{
    constexpr int NW = RG * KS, NT = 64 * NW;
    constexpr int NB = 16 * RBW * RG;
    constexpr int FM = MT / 16;                  // 16-token blocks
    constexpr bool PG = GS != 0;
    constexpr int UK = BITS == 8 ? 128 : 256;    // k values per unit
    constexpr int STEPS = UK / 64;               // 64-deep MFMA steps per unit
    constexpr int XP = UK / 128;                 // token lines per row and unit
    constexpr int GPU = PG ? UK / GS : 1;        // groups per unit
    constexpr int SPG = PG ? GS / 64 : STEPS;    // steps per group
    constexpr int SLOTS = RBW + FM * XP;         // 2 KB slots per wavefront
    constexpr int TS = NB + 1;                   // partial tile row stride (words)
    constexpr int PART = KS * MT * TS * 4;
    constexpr int LDS = NW * SLOTS * kSlot > PART ? NW * SLOTS * kSlot : PART;
    static_assert(!(PG && OUT == OUT_I32), "per-group int32 sums take the other kernels");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
    __shared__ float s_st[MT], s_sw[NB];

    const int64_t M = args.M, N = args.N, K = args.K;
    const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    const int64_t n0 = (int64_t)tn * NB, m0 = (int64_t)tm * MT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave % RG, ks = wave / RG;
    const int64_t wld = BITS == 8 ? K : K / 2;
    const int G = PG ? (int)(K / GS) : 1;
    const int KU = (int)(K / UK);
    const int nu = KU > ks ? (KU - ks + KS - 1) / KS : 0;  // this wavefront's units

    const auto rx = __builtin_amdgcn_make_buffer_rsrc((void *)args.xq, (short)0, (int)(M * K), kRsrcWord3);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc((void *)args.wq, (short)0, (int)(N * wld), kRsrcWord3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)args.s_w, (short)0,
                                                      (OUT != OUT_I32 && PG) ? (int)(N * G * 4) : 0, kRsrcWord3);

    // Dequantization scales of the tile, loaded now (their latency hides
    // under the main loop) and put into LDS before the reduction's barrier.
    constexpr int NSV = PG ? MT : MT + NB;
    constexpr int NSC = OUT != OUT_I32 ? (NSV + NT - 1) / NT : 0;
    float scv[NSC > 0 ? NSC : 1];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int o = (int)threadIdx.x + i * NT;
        const float *src = o < MT ? args.s_tok + min(m0 + o, M - 1)
                                  : args.s_w + min(n0 + min(o - MT, NB - 1), N - 1);
        scv[i] = *src;
    }

    // Line loads: lane l reads bytes 16 (l % 8) .. +15 of row 8 h + l / 8 of
    // a 16-row block (h = 0, 1); rows past the operand read zeros.
    const int lrow = lane >> 3, lcol = (lane & 7) * 16;
    uint32_t wrow[RBW][2], xrow[FM][2];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t n = n0 + 16 * (rg * RBW + i) + 8 * h + lrow;
            wrow[i][h] = n < N ? (uint32_t)(n * wld) + lcol : kDead;
        }
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t m = m0 + 16 * j + 8 * h + lrow;
            xrow[j][h] = m < M ? (uint32_t)(m * K) + lcol : kDead;
        }
    // group scales: lane l's channel in block i is 16 (rg RBW + i) + l % 16
    uint32_t srow[PG ? RBW : 1];
#pragma unroll
    for (int i = 0; i < (PG ? RBW : 1); ++i) {
        const int64_t n = n0 + 16 * (rg * RBW + i) + (lane & 15);
        srow[i] = (PG && n < N) ? (uint32_t)(n * G) * 4u : kDead;
    }

    struct Unit {
        i32x4 w[RBW][2];
        i32x4 x[FM][XP][2];
        float sw[PG ? RBW : 1][PG ? GPU : 1];
    };
    // Offsets past the wavefront's last unit get the top bit set (or kept):
    // beyond every operand, so those loads return zeros.  Branch-free, so the
    // memory counter waits stay exact.
    auto load_unit = [&](Unit &t, int ui) {  // ui: this wavefront's ui-th unit
        const uint32_t dead = ui < nu ? 0u : kDead;
        const uint32_t u = (uint32_t)(ks + ui * KS);
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                t.w[i][h] = load16<2>(rw, (wrow[i][h] + u * 128u) | dead);
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int p = 0; p < XP; ++p)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    t.x[j][p][h] = load16<0>(rx, (xrow[j][h] + u * UK + p * 128u) | dead);
        if constexpr (PG && OUT != OUT_I32) {
#pragma unroll
            for (int i = 0; i < RBW; ++i)
#pragma unroll
                for (int q = 0; q < GPU; ++q)
                    t.sw[i][q] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rs, (srow[i] + (u * GPU + q) * 4u) | dead, 0, 0));
        }
    };

    uint8_t *const mine = lds + wave * SLOTS * kSlot;
    // slot order: weight blocks 0..RBW-1, then token block j, line p
    auto put = [&](int slot, const i32x4 (&v)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<i32x4 *>(mine + slot * kSlot + slot_off(8 * h + lrow, lane & 7)) = v[h];
    };
    const int frow = lane & 15, fq = lane >> 4;  // fragment row, chunk within a 64-deep step
    auto frag8 = [&](int slot, int s) {  // int8 fragment of 64-deep step s (0, 1) of a line
        return *reinterpret_cast<const i32x4 *>(mine + slot * kSlot + slot_off(frow, 4 * s + fq));
    };
    auto frag4 = [&](int slot, int s) {  // int4 fragment of step s (0..3): 8 packed bytes, widened
        const uint2 p = *reinterpret_cast<const uint2 *>(mine + slot * kSlot + slot_off(frow, 2 * s + (fq >> 1)) +
                                                         8 * (fq & 1));
        uint32_t d0, d1, d2, d3;
        widen8(p.x, d0, d1);
        widen8(p.y, d2, d3);
        return i32x4{(int)d0, (int)d1, (int)d2, (int)d3};
    };

    i32x4 acc[RBW][FM];
    float facc[PG ? RBW : 1][PG ? FM : 1][PG ? 4 : 1];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            acc[i][j] = i32x4{};
            if constexpr (PG)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    facc[i][j][e] = 0.f;
        }

    // Ring entry r holds this wavefront's units r, r + R, ...; the prologue
    // issues entries in order (kept by the scheduling barriers), so entry 0
    // is always the oldest load in flight when its pass begins.
    Unit ring[R];
#pragma unroll
    for (int p = 0; p < R; ++p) {
        load_unit(ring[p], p);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int ub = 0; ub < nu; ub += R) {
        // Every pass runs all R ring entries: entries past the wavefront's
        // last unit hold zeros (their loads were dropped by the range check)
        // and add nothing.  A branch-free pass keeps the compiler's memory
        // counter waits exact (one unit's loads at a time), where an early
        // exit made it wait for every load in flight at the top of the pass.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int ui = ub + r;
            Unit &t = ring[r];
            // lines into the slots; the registers take unit ui + R at once
            // (the scheduling barriers keep this order: the compiler would
            // otherwise hoist every entry's slot writes, with a wait for all
            // loads in flight, above the refills)
#pragma unroll
            for (int i = 0; i < RBW; ++i)
                put(i, t.w[i]);
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int p = 0; p < XP; ++p)
                    put(RBW + j * XP + p, t.x[j][p]);
            float sw[PG ? RBW : 1][PG ? GPU : 1];
#pragma unroll
            for (int i = 0; i < (PG ? RBW : 1); ++i)
#pragma unroll
                for (int q = 0; q < (PG ? GPU : 1); ++q)
                    sw[i][q] = t.sw[i][q];
            __builtin_amdgcn_sched_barrier(0);
            load_unit(t, ui + R);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                i32x4 xf[FM], wf[RBW];
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    xf[j] = frag8(RBW + j * XP + s / 2, s % 2);
#pragma unroll
                for (int i = 0; i < RBW; ++i)
                    wf[i] = BITS == 8 ? frag8(i, s) : frag4(i, s);
#pragma unroll
                for (int i = 0; i < RBW; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        if constexpr (!PG)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], xf[j], acc[i][j], 0, 0, 0);
                        else if (s % SPG == 0)  // a group opens: start from zero
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[j], wf[i], i32x4{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[j], wf[i], acc[i][j], 0, 0, 0);
                    }
                if constexpr (PG) {
                    if (s % SPG == SPG - 1) {  // a group closes: scale it
#pragma unroll
                        for (int i = 0; i < RBW; ++i)
#pragma unroll
                            for (int j = 0; j < FM; ++j)
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    facc[i][j][e] += (float)acc[i][j][e] * sw[i][s / SPG];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Partial tiles [ks][token][channel] over the slots (every wavefront is
    // past its last fragment read after the barrier).  Block (i, j) gives the
    // lane: per channel, token 16j + lane%16 and channels 16i' + 4(lane/16) + e;
    // per group, channel 16i' + lane%16 and tokens 16j + 4(lane/16) + e
    // (i' = rg RBW + i).
    __syncthreads();
    int32_t *part = reinterpret_cast<int32_t *>(lds) + ks * MT * TS;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ci = 16 * (rg * RBW + i);
                if constexpr (!PG)
                    part[(16 * j + frow) * TS + ci + 4 * fq + e] = acc[i][j][e];
                else
                    part[(16 * j + 4 * fq + e) * TS + ci + frow] = __builtin_bit_cast(int32_t, facc[i][j][e]);
            }
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int o = (int)threadIdx.x + i * NT;
        if (o < MT)
            s_st[o] = scv[i];
        else if (o < NSV)
            s_sw[o - MT] = scv[i];
    }
    __syncthreads();

    // Sum the K-split partials in order, dequantize, store two outputs per
    // thread (consecutive channels; one at a time when N is odd).
    const int32_t *p0 = reinterpret_cast<const int32_t *>(lds);
    const bool pairs = (N & 1) == 0;
    for (int o = threadIdx.x; o < MT * NB / 2; o += NT) {
        const int t = o / (NB / 2), c = 2 * (o % (NB / 2));
        const int64_t m = m0 + t, n = n0 + c;
        if (m >= M || n >= N)
            continue;
        if constexpr (!PG) {
            int32_t s0 = 0, s1 = 0;
#pragma unroll
            for (int z = 0; z < KS; ++z) {
                s0 += p0[(z * MT + t) * TS + c];
                s1 += p0[(z * MT + t) * TS + c + 1];
            }
            if constexpr (OUT == OUT_I32) {
                int32_t *y = static_cast<int32_t *>(args.out) + m * N + n;
                y[0] = s0;
                if (n + 1 < N)
                    y[1] = s1;
            } else {
                const float y0 = (float)s0 * s_st[t] * s_sw[c];
                const float y1 = (float)s1 * s_st[t] * s_sw[c + 1];
                uint16_t *y = static_cast<uint16_t *>(args.out) + m * N + n;
                if (pairs) {
                    *reinterpret_cast<uint32_t *>(y) = pack2<OUT>(y0, y1);
                } else {
                    y[0] = out_bits<OUT>(y0);
                    if (n + 1 < N)
                        y[1] = out_bits<OUT>(y1);
                }
            }
        } else {
            float f0 = 0.f, f1 = 0.f;
#pragma unroll
            for (int z = 0; z < KS; ++z) {
                f0 += __builtin_bit_cast(float, p0[(z * MT + t) * TS + c]);
                f1 += __builtin_bit_cast(float, p0[(z * MT + t) * TS + c + 1]);
            }
            const float y0 = s_st[t] * f0, y1 = s_st[t] * f1;
            uint16_t *y = static_cast<uint16_t *>(args.out) + m * N + n;
            if (pairs) {
                *reinterpret_cast<uint32_t *>(y) = pack2<OUT>(y0, y1);
            } else {
                y[0] = out_bits<OUT>(y0);
                if (n + 1 < N)
                    y[1] = out_bits<OUT>(y1);
            }
        }
    }
}

template <int BITS, int GS, int OUT, int MT, int RBW, int RG, int KS, int R>
hipError_t launch_cfg(const ProductArgs &a, hipStream_t stream)
{
    constexpr int NB = 16 * RBW * RG;
    const int tiles_n = (int)((a.N + NB - 1) / NB);
    const int tiles_m = (int)((a.M + MT - 1) / MT);
    hipLaunchKernelGGL((few_kernel<BITS, GS, OUT, MT, RBW, RG, KS, R>), dim3(tiles_n * tiles_m),
                       dim3(64 * RG * KS), 0, stream, a, tiles_n);
    return hipGetLastError();
}

// Tile shapes (RBW blocks per wavefront, RG row groups, KS K-splits), each
// with two units in flight per wavefront: deeper rings measured slower (int8
// per channel, M = 16: 8.6 / 8.7 / 9.9 / 9.9 us at 2 / 3 / 4 / 6 units; one
// unit as fast as two), as the token loads then queue behind more weight
// lines.  Per channel at N >= 8192, 64-channel tiles: up to 16 tokens four
// row groups of one block over two K-splits, up to 32 tokens (int8) one
// wavefront of four blocks per K-split, four K-splits, or (int4) two row
// groups of two blocks over two; otherwise 16-channel tiles over eight
// K-splits (int4 per group: four).  Measured at N = 10240, K = 2560 and
// N = 2560, K = 10240 against the other shapes tried (64-channel tiles of
// 2 x 2 x 4, 32-channel tiles, 16 wavefronts).
constexpr int kRing = 2;

template <int BITS, int GS, int OUT, int MT>
hipError_t launch_mt(const ProductArgs &a, hipStream_t stream)
{
    if constexpr (GS == 0) {
        if (a.N >= 8192) {
            if constexpr (MT == 16)
                return launch_cfg<BITS, GS, OUT, MT, 1, 4, 2, kRing>(a, stream);
            else if constexpr (BITS == 8)
                return launch_cfg<BITS, GS, OUT, MT, 4, 1, 4, kRing>(a, stream);
            else
                return launch_cfg<BITS, GS, OUT, MT, 2, 2, 2, kRing>(a, stream);
        }
    }
    if constexpr (GS != 0 && BITS == 4)
        return launch_cfg<BITS, GS, OUT, MT, 1, 1, 4, kRing>(a, stream);
    else
        return launch_cfg<BITS, GS, OUT, MT, 1, 1, 8, kRing>(a, stream);
}

template <int BITS, int GS, int OUT>
hipError_t launch_out(const ProductArgs &a, hipStream_t stream)
{
    if (a.M <= 16)
        return launch_mt<BITS, GS, OUT, 16>(a, stream);
    return launch_mt<BITS, GS, OUT, 32>(a, stream);
}

template <int BITS, int GS>
hipError_t launch_gs(const ProductArgs &a, hipStream_t stream)
{
    switch (a.out_kind) {
    case OUT_F16: return launch_out<BITS, GS, OUT_F16>(a, stream);
    case OUT_BF16: return launch_out<BITS, GS, OUT_BF16>(a, stream);
    default:
        if constexpr (GS == 0)
            return launch_out<BITS, GS, OUT_I32>(a, stream);
        else
            return hipErrorNotSupported;
    }
}

}  // namespace

bool few_shape_ok(const ProductArgs &a)
{
    const int64_t uk = a.bits == 8 ? 128 : 256;
    const int64_t wld = a.bits == 8 ? a.K : a.K / 2;
    const int64_t G = a.group_size ? a.K / a.group_size : 1;
    return a.M >= 1 && a.N >= 1 && a.K >= uk && a.K % uk == 0 &&
           !(a.group_size != 0 && a.out_kind == OUT_I32) && a.N * wld < (1LL << 31) &&
           (a.M + 32) * a.K < (1LL << 31) && a.N * G * 4 < (1LL << 31);
}

bool few_supported(const ProductArgs &a) { return a.M <= 32 && few_shape_ok(a); }

hipError_t launch_gemm_few(const ProductArgs &a, hipStream_t stream)
{
    if (!few_shape_ok(a))
        return hipErrorNotSupported;
    if (a.bits == 8) {
        if (a.group_size == 0)
            return launch_gs<8, 0>(a, stream);
        return a.group_size == 64 ? launch_gs<8, 64>(a, stream) : launch_gs<8, 128>(a, stream);
    }
    if (a.group_size == 0)
        return launch_gs<4, 0>(a, stream);
    return a.group_size == 64 ? launch_gs<4, 64>(a, stream) : launch_gs<4, 128>(a, stream);
}

}  // namespace cider
