// Pipelined matrix-core product for all three modes: W8A8 per channel, W8A8
// per group of 64 / 128 along K, and W4A8 (Cider README, ossradar.top repo
// page, "Quantization" table: INT32 accumulation, C_fp16 = C_int32 * s_act *
// s_weight per element; "W8A8 Quantization Granularity": one scale per
// output channel or per group; "Modes": W4A8 unpacks INT4 before the INT8
// product; "TensorOps matmul2d": dequantization fused into the store phase).
//
// Structure (gfx950):
//   * v_mfma_i32_32x32x32_i8; per channel the weight tile is operand A and
//     the token tile operand B (a lane's outputs are 4 consecutive channels
//     of one token); per group the roles swap (a lane's outputs are 16
//     tokens of one channel, so each group needs one scale per lane and
//     32-channel block).  A wavefront owns WN x WM outputs.
//   * K advances BK bytes per tile (64; 128 or 256 for few tokens).  Tiles go
//     from HBM to LDS with
//     buffer_load_dwordx4 ... lds (no registers involved) through a ring of
//     STAGES LDS stages, so STAGES - 1 tiles of copies are in flight while
//     the matrix cores work; a tile's copies are awaited with a counted
//     vmcnt, not a full drain.  Per group, the tile's channel scales of its
//     group travel the same way (buffer_load_dword ... lds).
//   * Each tile is BK / 32 matrix-core steps of 32.  The fragments of the
//     next step are read from LDS while the current step's MFMAs run (two
//     register sets, reads interleaved between MFMAs).  The one barrier per
//     tile sits before the last step, where the queued MFMAs cover it; the
//     stage consumed by the previous tile is refilled around it.
//   * Per group, a group's first MFMA starts from zero and, once its last
//     K tile is multiplied, its int32 sums are scaled into fp32 accumulators.
//   * int8 tiles: rows of 64 bytes, 16-byte chunk c of row r at slot
//     c ^ (((r >> 1) ^ (r >> 2)) & 3), conflict-free for the fragment reads.
//     Packed int4 tiles: rows of 32 bytes, chunk c at slot c ^ ((r >> 3) & 1);
//     a lane reads 8 packed bytes and widens them to 16 int8 codes in
//     registers, so no unpacked copy of the weight tile is ever stored.
//   * Out-of-range rows read as zeros (buffer descriptors bound the operand);
//     their outputs are not stored.
#include "cider_kernels.h"

namespace cider {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kXcds = 8;

// LDS slot of 16-byte chunk `chunk` of int8 tile row `row` (rows of BK
// bytes).  Conflict-free for 16-byte reads of 32 consecutive rows at one
// chunk, whether LDS serves 8 lanes per 128 bytes or 16 lanes per 256 bytes.
template <int BK>
__device__ __forceinline__ int swz8(int row)
{
    return BK == 64 ? (((row >> 1) ^ (row >> 2)) & 3) : ((row & 7) ^ ((row >> 3) & 1));
}
template <int BK>
__device__ __forceinline__ int off8(int row, int chunk)
{
    return row * BK + ((chunk ^ swz8<BK>(row)) << 4);
}
// Packed int4 rows of BK/2 bytes.
template <int BK>
__device__ __forceinline__ int swz4(int row)
{
    return BK == 64 ? ((row >> 3) & 1) : (((row >> 1) ^ (row >> 2)) & 3);
}
template <int BK>
__device__ __forceinline__ int off4(int row, int chunk)
{
    return row * (BK / 2) + ((chunk ^ swz4<BK>(row)) << 4);
}

// Raw buffer resource (gfx9 layout, stride 0): byte offsets, loads at or
// past `bytes` return 0.  Kept in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void *p, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// One wavefront-wide asynchronous copy of 64 x 16 bytes from global memory
// straight into LDS: lane l's 16 bytes land at LDS address lds + 16 * l.
// Written as an instruction of its own because the compiler, seeing an LDS
// write it cannot disambiguate, would otherwise drain every copy in flight
// before each later LDS read; ordering against readers is enforced here by
// the counted vmcnt waits and barriers of the pipeline instead.  There is no
// register result: the data goes to LDS, and the operands are read at issue.
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(lds_void_t *)p;
}

__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t lds_block, uint32_t voffset)
{
    const int lds = __builtin_amdgcn_readfirstlane((int)lds_block);
    int saved;  // m0 is left exactly as the compiler had it
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory");
}

// The same with the non-temporal cache policy, for operands that stream
// through once (the weights of a few-token product).
__device__ __forceinline__ void dma16_stream(const i32x4 &rsrc, uint32_t lds_block, uint32_t voffset)
{
    const int lds = __builtin_amdgcn_readfirstlane((int)lds_block);
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory");
}

// The same with 4 bytes per lane: lane l's dword lands at lds + 4 * l.
__device__ __forceinline__ void dma4(const i32x4 &rsrc, uint32_t lds_block, uint32_t voffset)
{
    const int lds = __builtin_amdgcn_readfirstlane((int)lds_block);
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "buffer_load_dword %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory");
}

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most n * DT copies are in flight, n (wavefront-uniform)
// clamped to 0 .. MAXN.
template <int DT, int MAXN>
__device__ __forceinline__ void wait_tiles(int n)
{
    if constexpr (MAXN <= 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= MAXN)
            wait_vmcnt<MAXN * DT>();
        else
            wait_tiles<DT, MAXN - 1>(n);
    }
}

__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Widen 8 packed nibbles (low nibble = even k) to int8 codes q = u - 8, k
// order kept: the even-k nibbles (low) and odd-k nibbles (high) are masked
// into bytes, interleaved with two byte permutes, and each byte u becomes
// u - 8 as (u + 0x78) ^ 0x80 (no carry leaves a byte for u <= 15).  Nine VALU
// operations per 8 codes: the int4 product's main loop is otherwise bound by
// this widening, not by the matrix cores.
__device__ __forceinline__ void unpack8(uint32_t v, uint32_t &d0, uint32_t &d1)
{
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // k0 k1 k2 k3
    const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // k4 k5 k6 k7
    d0 = (a + 0x78787878u) ^ 0x80808080u;
    d1 = (b + 0x78787878u) ^ 0x80808080u;
}

// The same nibbles as unsigned bytes u = q + 8 (five operations per 8
// codes).  Per channel the product takes these and subtracts 8 * sum_k x[m, k]
// per token once the K loop is done: sum q x = sum u x - 8 sum x, exactly in
// int32 (|sum u x| <= 15 * 127 * K).
__device__ __forceinline__ void unpack8u(uint32_t v, uint32_t &d0, uint32_t &d1)
{
    const uint32_t lo = v & 0x0F0F0F0Fu;
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
    d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

__device__ __forceinline__ void tile_coords(int pid, int tiles_n, int tiles_m, int group_m,
                                            int &tn, int &tm)
{
    const int total = tiles_n * tiles_m;
    int logical = pid;
    if (total % kXcds == 0) {
        const int per = total / kXcds;
        logical = (pid % kXcds) * per + pid / kXcds;
    }
    const int in_group = group_m * tiles_n;
    const int gid = logical / in_group;
    const int first_m = gid * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int r = logical - gid * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// GS = 0: one scale per channel.  GS = 64 / 128: per-group scaling.  The
// operands then swap roles -- tokens are operand A, weights operand B -- so
// that a lane's outputs all belong to one channel per 32-channel block and
// need one group scale each; the int32 sum of each group is scaled into an
// fp32 accumulator as soon as the group's last K tile is multiplied.
// SPLIT: workgroup blockIdx.x computes split z = blockIdx.x / tiles of tile
// blockIdx.x % tiles (the splits of a tile share its XCD), over its share
// of the K tiles, then takes part in the split reduction.
template <int TN, int TM, int WN, int WM, int BK, int BITS, int GS, int OUT, int STAGES, bool SPLIT = false>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_kernel(
    ProductArgs args, int tiles_n, int tiles_m, int group_m, SplitArgs sp)
{
    constexpr int NWN = TN / WN, NWM = TM / WM, NW = NWN * NWM;
    constexpr int FN = WN / 32, FM = WM / 32;
    constexpr int KSTEPS = BK / 32;
    static_assert(KSTEPS % 2 == 0, "an even number of 32-deep steps per tile");
    constexpr bool PG = GS != 0;
    static_assert(!PG || GS == BK || GS == 2 * BK, "a group spans one or two K tiles");
    constexpr int XROW = BK, WROW = BITS == 8 ? BK : BK / 2;        // bytes per tile row
    constexpr int XBYTES = TM * XROW, WBYTES = TN * WROW;            // per stage
    // Per group with the fp16 epilogue: the tile's TN channel scales of the
    // tile's group, one dword each, copied with the operands (256-byte
    // blocks), padded to 1 KB.  The int32 hook has no scales (s_w is null):
    // no scale copies at all.
    constexpr bool SCOPY = PG && OUT != OUT_I32;
    constexpr int SB = SCOPY ? (TN * 4 + 255) / 256 : 0;  // the last block may run past TN
    constexpr int SBYTES = SCOPY ? (SB * 256 + 1023) / 1024 * 1024 : 0;
    constexpr int STAGE = XBYTES + WBYTES + SBYTES;
    constexpr int XB = XBYTES / 1024, WB = WBYTES / 1024;            // 1 KB copy blocks
    constexpr int TB = XB + WB;
    // Copies per wave per tile.  When the blocks do not split evenly, the
    // last slots repeat the final block (identical bytes to the same place),
    // so every wave issues the same number and vmcnt counts stay uniform.
    constexpr int D = (TB + NW - 1) / NW;
    constexpr int DS = SCOPY ? (SB + NW - 1) / NW : 0;  // scale copies per wave per tile
    constexpr int DT = D + DS;
    static_assert(XBYTES % 1024 == 0 && WBYTES % 1024 == 0, "tiles of whole 1 KB blocks");
    static_assert(STAGES >= 2 && (STAGES - 1) * DT < 64, "vmcnt range");

    // The fp16 per-channel epilogue reuses the stage ring to stage its rows
    // (rows of 2 * WN bytes padded by 16); it may need more than the ring.
    constexpr int ROWB = WN * 2 + 16;
    constexpr int OSTAGE = OUT != OUT_I32 && !PG ? NW * 32 * ROWB : 0;
    constexpr int SMEM = STAGES * STAGE > OSTAGE ? STAGES * STAGE : OSTAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    __shared__ __attribute__((aligned(16))) float s_sw[OUT != OUT_I32 && !PG ? TN : 4];  // s_w tile
    __shared__ __attribute__((aligned(16))) float s_st[OUT != OUT_I32 ? TM : 4];         // s_tok tile

    const int64_t M = args.M, N = args.N, K = args.K;
    int pid = blockIdx.x, z = 0;
    if constexpr (SPLIT) {
        z = pid / (tiles_n * tiles_m);
        pid -= z * (tiles_n * tiles_m);
    }
    int tn, tm;
    tile_coords(pid, tiles_n, tiles_m, group_m, tn, tm);
    const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWN, wm = wave / NWN;
    const uint32_t wld = (uint32_t)(BITS == 8 ? K : K / 2);
    // This workgroup's K tiles kt0 .. kt0 + KT - 1 (a split takes whole
    // groups; the host guarantees every split at least one).
    int kt0 = 0, KT = (int)(K / BK);
    if constexpr (SPLIT) {
        constexpr int U = PG ? GS / BK : 1;
        const int KU = KT / U;
        const int u0 = (int)((int64_t)z * KU / sp.splits), u1 = (int)((int64_t)(z + 1) * KU / sp.splits);
        kt0 = u0 * U;
        KT = (u1 - u0) * U;
    }

    const i32x4 rX = make_rsrc(args.xq, (uint32_t)(M * K));
    const i32x4 rW = make_rsrc(args.wq, (uint32_t)(N * (int64_t)wld));
    const int G = PG ? (int)(K / GS) : 1;

    // Source offset of this lane's 16 bytes in each of the wave's copy blocks,
    // and the block's LDS offset within a stage.  Blocks 0 .. XB-1 hold token
    // rows, the rest weight rows; LDS slot s of row r receives global chunk
    // s ^ swizzle(r).
    constexpr int CX = XROW / 16, CW = WROW / 16;  // 16-byte chunks per row
    uint32_t coff[D], cstep[D];
    int cdst[D];
    i32x4 crs[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int b = min(wave * D + j, TB - 1);  // wavefront-uniform
        crs[j] = b < XB ? rX : rW;
        cstep[j] = b < XB ? XROW : WROW;
        if (b < XB) {
            const int r = b * (1024 / XROW) + lane / CX, c = (lane % CX) ^ swz8<BK>(r);
            coff[j] = (uint32_t)((m0 + r) * K) + c * 16;
            cdst[j] = b * 1024;
        } else {
            const int bw = b - XB;
            const int r = bw * (1024 / WROW) + lane / CW;
            const int c = (lane % CW) ^ (BITS == 8 ? swz8<BK>(r) : swz4<BK>(r));
            coff[j] = (uint32_t)((n0 + r) * (int64_t)wld) + c * 16;
            cdst[j] = XBYTES + bw * 1024;
        }
    }
    // Scale copies: block sb holds channels n0 + 64 sb .. +63; lane l reads
    // s_w[n0 + 64 sb + l, g] (past N: out of range, reads 0).
    const i32x4 rS = SCOPY ? make_rsrc(args.s_w, (uint32_t)(N * G * 4)) : rX;
    uint32_t soff[DS > 0 ? DS : 1];
    int sdst[DS > 0 ? DS : 1];
#pragma unroll
    for (int j = 0; j < DS; ++j) {
        const int sb = min(wave * DS + j, SB - 1);  // wavefront-uniform
        soff[j] = (uint32_t)((n0 + sb * 64 + lane) * G) * 4u;
        sdst[j] = XBYTES + WBYTES + sb * 256;
    }
    // Copy instruction j (0 <= j < DT) of this wave's share of tile `src`
    // into LDS stage `stage`: operand blocks, then scale blocks.
    const uint32_t smem_lds = lds_address(smem);
    // Tiles of up to 32 tokens with deep K tiles or split K read each weight
    // byte once: those copies are non-temporal (M = 16 / 32 per channel:
    // 7-8% faster; with 64- and 128-token tiles they measured slower).
    constexpr bool STREAM_W = TM <= 32 && (SPLIT || BK > 64);
    auto copy_one = [&](int j, int stage, int src) {
        if (j < D) {
            const uint32_t dst = smem_lds + stage * STAGE + cdst[j], off = coff[j] + (uint32_t)(kt0 + src) * cstep[j];
            if (STREAM_W && cdst[j] >= XBYTES)  // a weight block (wavefront-uniform)
                dma16_stream(crs[j], dst, off);
            else
                dma16(crs[j], dst, off);
        } else if constexpr (SCOPY) {
            const uint32_t g = (uint32_t)((kt0 + src) * BK / GS);
            dma4(rS, smem_lds + stage * STAGE + sdst[j - D], soff[j - D] + g * 4u);
        }
    };

    // Fragment register sets: a = weight rows (operand A, int8 codes; for
    // int4 the packed bytes sit in ap until widened), b = token rows.
    struct Frags {
        i32x4 a[FN];
        uint2 ap[BITS == 4 ? FN : 1];
        i32x4 b[FM];
    };
    const int frow = lane & 31, fhalf = lane >> 5;
    constexpr int LOADS = FN + FM;
    // Fragment read k: weight fragments first, then token fragments.
    auto load_one = [&](Frags &f, int k, int kt, int ks) {
        const uint8_t *st = smem + (kt % STAGES) * STAGE;
        if (k < FN) {
            const int r = wn * WN + k * 32 + frow;
            if constexpr (BITS == 8)
                f.a[k] = *reinterpret_cast<const i32x4 *>(st + XBYTES + off8<BK>(r, ks * 2 + fhalf));
            else
                f.ap[k] = *reinterpret_cast<const uint2 *>(st + XBYTES + off4<BK>(r, ks) + fhalf * 8);
        } else {
            const int j = k - FN;
            f.b[j] = *reinterpret_cast<const i32x4 *>(st + off8<BK>(wm * WM + j * 32 + frow, ks * 2 + fhalf));
        }
    };
    // int4 per channel: unsigned codes, corrected by the token sums below.
    constexpr bool USUM = BITS == 4 && !PG;
    auto widen = [&](Frags &f, int i) {
        if constexpr (BITS == 4) {
            uint32_t d0, d1, d2, d3;
            if constexpr (USUM) {
                unpack8u(f.ap[i].x, d0, d1);
                unpack8u(f.ap[i].y, d2, d3);
            } else {
                unpack8(f.ap[i].x, d0, d1);
                unpack8(f.ap[i].y, d2, d3);
            }
            f.a[i] = i32x4{(int)d0, (int)d1, (int)d2, (int)d3};
        }
    };
    // Sums of the token codes this lane multiplies: token block j's row
    // (lane % 32), the 16-byte chunks of half lane / 32 of every step.
    int xs[USUM ? FM : 1];
#pragma unroll
    for (int j = 0; j < (USUM ? FM : 1); ++j)
        xs[j] = 0;

    i32x16 acc[FN][FM];
    // Per group (fp16 output): facc accumulates each group's int32 sums
    // times the group's channel scales, in group order.
    constexpr bool SCALED = PG && OUT != OUT_I32;
    float facc[SCALED ? FN : 1][SCALED ? FM : 1][SCALED ? 16 : 1];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            acc[i][j] = i32x16{};
            if constexpr (SCALED)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    facc[i][j][e] = 0.f;
        }

    // One 32-deep step: `copies` copy instructions first (a short burst; the
    // other wavefront on the SIMD keeps the matrix core busy meanwhile), then
    // the FN x FM MFMAs on `cur` with the LOADS fragment reads of the next
    // step (into `nxt`) spread between them by the scheduler.  `first`: the
    // step opens a group (per group only), so the MFMAs start from zero.
    auto step = [&](auto first, Frags &cur, Frags &nxt, int lkt, int lks, int copies, int cstart,
                    int cstage, int csrc) {
        constexpr int MF = FN * FM;
#pragma unroll
        for (int c = 0; c < 12; ++c)
            if (c < copies)
                copy_one(cstart + c, cstage, csrc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < LOADS; ++k)
            load_one(nxt, k, lkt, lks);
        if constexpr (USUM) {
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xs[j] = __builtin_amdgcn_sdot4(cur.b[j][e], 0x01010101, xs[j], false);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            widen(cur, i);
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                if constexpr (!PG) {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
                } else if constexpr (decltype(first)::value) {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.b[j], cur.a[i], i32x16{}, 0, 0, 0);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
                }
            }
        }
        constexpr int PER = MF / LOADS > 0 ? MF / LOADS : 1;
#pragma unroll
        for (int k = 0; k < LOADS; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // then MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // The dequant scales of this tile's channels and tokens go into registers
    // now (branch-free loads whose latency hides under the main loop) and
    // into LDS only before the epilogue: storing them to LDS here would make
    // every wave wait for them before it issues its first copy.  Indices are
    // clamped into range; values past the edge are never used.
    constexpr int TSW = PG ? 0 : TN;  // per group, channel scales come with the tiles
    constexpr int NSC = OUT != OUT_I32 ? (TSW + TM + NW * 64 - 1) / (NW * 64) : 0;
    float scv[NSC > 0 ? NSC : 1];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int t = (int)threadIdx.x + i * NW * 64;
        const float *src = t < TSW ? args.s_w + min(n0 + t, N - 1)
                                   : args.s_tok + min(m0 + min(t - TSW, TM - 1), M - 1);
        scv[i] = *src;
    }

    // Ring of STAGES stages.  Tile kt is computed from stage kt % STAGES;
    // while it runs, tile kt + STAGES - 1 is copied into the stage tile kt-1
    // used (free since tile kt-1's barrier), half of its copies during each
    // of the two steps, so the vmcnt bound at each barrier is a constant.
    // The last STAGES - 1 tiles issue no copies and wait for what is left
    // of the ring.  (When K has fewer than STAGES - 1 tiles, the prologue
    // repeats tile KT-1 into stages nobody reads; the waits below then only
    // count conservatively.)
    static_assert(KSTEPS == 2 || !PG, "per group, two 32-deep steps per tile");
    static_assert(STAGES >= 3, "the refill targets the stage freed one tile earlier");
    constexpr int DA = D / 2;
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
#pragma unroll
        for (int j = 0; j < DT; ++j)
            copy_one(j, p, min(p, KT - 1));
    wait_vmcnt<(STAGES - 2) * DT>();  // tile 0 has landed
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
#pragma unroll
    for (int k = 0; k < LOADS; ++k)
        load_one(f0, k, 0, 0);

    // Tile kt.  Per group: `first` opens a group, `last` closes it (its int32
    // sums are then scaled into facc, or stored by the int32 hook).
    auto tile = [&](int kt, auto first, auto last) {
        const int rstage = (kt + STAGES - 1) % STAGES;  // == (kt - 1) mod STAGES
        const int rsrc = min(kt + STAGES - 1, KT - 1);
        // the closing group's scales, read while tile kt's stage is intact
        float sw[SCALED ? FN : 1];
        if constexpr (SCALED && decltype(last)::value) {
            const float *ss = reinterpret_cast<const float *>(smem + (kt % STAGES) * STAGE + XBYTES + WBYTES);
#pragma unroll
            for (int i = 0; i < FN; ++i)
                sw[i] = ss[wn * WN + i * 32 + frow];
        }
        const bool refill = kt + STAGES - 1 < KT;  // wavefront-uniform
        // step 0: reads step 1's fragments, first half of the refill
        step(first, f0, f1, kt, 1, refill ? DA : 0, 0, rstage, rsrc);
        // deeper tiles: the middle steps, each reading the next step's
        // fragments from the same stage (the register sets alternate)
#pragma unroll
        for (int ks = 1; ks < KSTEPS - 1; ks += 2) {
            step(Flag<false>{}, f1, f0, kt, ks + 1, 0, 0, rstage, rsrc);
            step(Flag<false>{}, f0, f1, kt, ks + 2, 0, 0, rstage, rsrc);
        }
        // Tile kt+1 must have landed; tiles kt+2 .. kt+STAGES-2 and the first
        // half of tile kt+STAGES-1 may still be in flight (in the last tiles:
        // tiles kt+2 .. KT-1).  Every wave must also be done reading tile
        // kt's stage (its last fragments were read in the step just run)
        // before anyone refills it.
        wait_lgkm0();
        if (refill)
            wait_vmcnt<(STAGES - 3) * DT + DA>();
        else
            wait_tiles<DT, STAGES - 3>(KT - 2 - kt);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // last step: reads tile kt+1's step-0 fragments (at the last tile: a
        // stage whose contents are never used), second half of the refill
        step(Flag<false>{}, f1, f0, kt + 1, 0, refill ? DT - DA : 0, DA, rstage, rsrc);
        if constexpr (PG && decltype(last)::value) {
            if constexpr (SCALED) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            facc[i][j][e] += (float)acc[i][j][e] * sw[i];
            } else {
                // int32 hook: acc[m, n, g] for this lane's channel and tokens
                const int64_t g = (int64_t)(kt0 + kt) * BK / GS;
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int64_t n = n0 + wn * WN + i * 32 + frow;
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int64_t m = m0 + wm * WM + j * 32 + (e / 4) * 8 + fhalf * 4 + e % 4;
                            if (m < M && n < N)
                                static_cast<int32_t *>(args.out)[(m * N + n) * G + g] = acc[i][j][e];
                        }
                }
                wait_vmcnt<0>();  // keep the copy counts exact: no store left in flight
            }
        }
    };
    if constexpr (!PG) {
        for (int kt = 0; kt < KT; ++kt)
            tile(kt, Flag<false>{}, Flag<false>{});
    } else if constexpr (GS == BK) {
        for (int kt = 0; kt < KT; ++kt)
            tile(kt, Flag<true>{}, Flag<true>{});
    } else {
        for (int kt = 0; kt < KT; kt += 2) {
            tile(kt, Flag<true>{}, Flag<false>{});
            tile(kt + 1, Flag<false>{}, Flag<true>{});
        }
    }

    if constexpr (USUM) {
        // both halves of each token's K: sum q x = sum u x - 8 sum x
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int t = 8 * (xs[j] + __shfl_xor(xs[j], 32, 64));
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i][j][e] -= t;
        }
    }

    // Nothing may still be landing in the ring (the prologue's repeats of a
    // short K) when the epilogue reuses it or the workgroup's LDS is handed
    // to the next workgroup.
    wait_vmcnt<0>();
    if constexpr (SPLIT) {
        // Split reduction.  Partial sums live tile by tile, split by split,
        // each lane's 16-byte quarters of its (i, j) block 64 lanes apart.
        // They are stored and loaded as relaxed device-scope atomics, which
        // this GPU performs at the device-coherent level, past the XCD-private
        // L2 caches; each split waits for its stores to complete before the
        // barrier after which thread 0 counts the split in, and the last of a
        // tile's splits to count in loads the others' partials only after
        // that.  (A release / acquire fence pair per workgroup would write
        // back and invalidate the whole L2 of its XCD instead -- measured at
        // 3-4x the time of the unsplit product.)  The partials are added in
        // split order, so the sum does not depend on which split was last.
        static_assert(OUT != OUT_I32, "split products dequantize");
        constexpr int TILE = TM * TN;
        typedef unsigned long long u64;
        uint32_t *mine = static_cast<uint32_t *>(sp.part) + (int64_t)pid * sp.splits * TILE +
                         wave * (64 * FN * FM * 16) + lane * 4;
        auto slot = [&](int zz, int i, int j, int q) {
            return reinterpret_cast<u64 *>(mine + (int64_t)zz * TILE + ((i * FM + j) * 4 + q) * 256);
        };
        auto quarter = [&](int i, int j, int q) -> i32x4 {
            if constexpr (SCALED)
                return i32x4{__float_as_int(facc[i][j][4 * q]), __float_as_int(facc[i][j][4 * q + 1]),
                             __float_as_int(facc[i][j][4 * q + 2]), __float_as_int(facc[i][j][4 * q + 3])};
            else
                return i32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        };
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const i32x4 v = quarter(i, j, q);
                    u64 *d = slot(z, i, j, q);
                    __hip_atomic_store(d, (u64)(uint32_t)v[0] | ((u64)(uint32_t)v[1] << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(d + 1, (u64)(uint32_t)v[2] | ((u64)(uint32_t)v[3] << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
        wait_vmcnt<0>();  // this lane's partial stores have completed
        __syncthreads();
        uint32_t *flag = reinterpret_cast<uint32_t *>(smem);  // the ring is idle now
        if (threadIdx.x == 0)
            *flag = __hip_atomic_fetch_add(sp.cnt + pid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*flag != (uint32_t)(sp.splits - 1))
            return;
        // Every split's partial (this one's included) is read back, split
        // after split, the next split's loads in flight while the previous
        // one is added (branch-free: past the last split the index is
        // clamped and the extra loads are not used).
        typedef i32x4 Part[FN][FM][4];
        auto fetch = [&](int zz, Part &dst) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u64 *src = slot(zz, i, j, q);
                        const u64 lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const u64 hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        dst[i][j][q] = i32x4{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi,
                                             (int)(uint32_t)(hi >> 32)};
                    }
        };
        auto add = [&](bool first_split, const Part &v) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (SCALED) {
                                const float f = __int_as_float(v[i][j][q][e]);
                                facc[i][j][4 * q + e] = first_split ? f : facc[i][j][4 * q + e] + f;
                            } else {
                                const int t = v[i][j][q][e];
                                acc[i][j][4 * q + e] = first_split ? t : acc[i][j][4 * q + e] + t;
                            }
                        }
        };
        const int S = sp.splits;
        Part pa, pb;
        fetch(0, pa);
        for (int zz = 0; zz < S; zz += 2) {
            fetch(min(zz + 1, S - 1), pb);
            add(zz == 0, pa);
            fetch(min(zz + 2, S - 1), pa);
            if (zz + 1 < S)
                add(false, pb);
        }
        // (every wave reads the flag before the barrier below, after which
        // the epilogue may reuse the ring)
    }
    if constexpr (OUT != OUT_I32) {
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int t = (int)threadIdx.x + i * NW * 64;
            if (t < TSW)
                s_sw[t] = scv[i];
            else if (t < TSW + TM)
                s_st[t - TSW] = scv[i];
        }
        __syncthreads();  // the scales are in LDS; every wave is done with the operand stages
    }

    // Epilogue.  Block (i, j) gives the lane token m = wm*WM + 32j + lane%32
    // and, for q = 0..3, output channels nb .. nb+3, nb = wn*WN + 32i + 8q +
    // 4*(lane/32).
    const bool full = m0 + TM <= M && n0 + TN <= N;  // uniform across the workgroup
    if constexpr (PG && OUT == OUT_I32) {
        // stored group by group above
    } else if constexpr (PG) {
        // Block (i, j): channel n = wn*WN + 32i + lane%32, tokens
        // wm*WM + 32j + 8q + 4*(lane/32) + e.  Two-byte stores; each
        // instruction writes two 64-byte runs of a token row.
        uint16_t *yout = static_cast<uint16_t *>(args.out);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int64_t n = n0 + wn * WN + i * 32 + frow;
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = wm * WM + j * 32 + (e / 4) * 8 + fhalf * 4 + e % 4;
                    const int64_t m = m0 + t;
                    const float y = s_st[t] * facc[i][j][e];
                    if (full || (m < M && n < N))
                        __builtin_nontemporal_store(out_bits<OUT>(y), yout + m * N + n);
                }
        }
    } else if constexpr (OUT == OUT_I32) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int64_t m = m0 + wm * WM + j * 32 + frow;
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t nb = n0 + wn * WN + i * 32 + q * 8 + fhalf * 4;
                    if (full || (m < M && nb < N)) {
                        const i32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        *reinterpret_cast<i32x4 *>(static_cast<int32_t *>(args.out) + m * N + nb) = v;
                    }
                }
        }
    } else {
        // fp16 results go through this wave's own LDS region one 32-token
        // block at a time: rows of 2*WN bytes padded by 16 (so the 32 rows a
        // write instruction touches fall in distinct bank groups), then leave
        // as 16-byte non-temporal stores, consecutive lanes along a token row
        // (5% faster at M = 8192 than stores that allocate in the caches).
        constexpr int CPRO = WN * 2 / 16;
        uint8_t *ob = smem + wave * (32 * ROWB);
        uint16_t *yout = static_cast<uint16_t *>(args.out);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const float st = s_st[wm * WM + j * 32 + frow];
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = i * 32 + q * 8 + fhalf * 4;  // channel within the wave tile
                    const f32x4 sw = *reinterpret_cast<const f32x4 *>(&s_sw[wn * WN + c]);
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = (float)acc[i][j][4 * q + e] * st * sw[e];
                    uint2 packed;
                    packed.x = (uint32_t)out_bits<OUT>(y[0]) | ((uint32_t)out_bits<OUT>(y[1]) << 16);
                    packed.y = (uint32_t)out_bits<OUT>(y[2]) | ((uint32_t)out_bits<OUT>(y[3]) << 16);
                    *reinterpret_cast<uint2 *>(ob + frow * ROWB + c * 2) = packed;
                }
            constexpr int CHUNKS = 32 * CPRO;
#pragma unroll
            for (int it = 0; it < (CHUNKS + 63) / 64; ++it) {
                const int id = it * 64 + lane;
                if (CHUNKS % 64 == 0 || id < CHUNKS) {
                    const int r = id / CPRO, c = id % CPRO;
                    const uint4 v = *reinterpret_cast<const uint4 *>(ob + r * ROWB + c * 16);
                    const int64_t m = m0 + wm * WM + j * 32 + r;
                    const int64_t n = n0 + wn * WN + c * 8;
                    if (full || (m < M && n < N))  // streaming store: Y is not read again here
                        __builtin_nontemporal_store(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                                    reinterpret_cast<i32x4 *>(yout + m * N + n));
                }
            }
        }
    }
}

template <int TN, int TM, int WN, int WM, int BK, int BITS, int GS, int OUT, int STAGES>
hipError_t launch_cfg(const ProductArgs &a, hipStream_t stream)
{
    if (a.K % BK != 0)  // the kernel walks whole K tiles
        return hipErrorInvalidValue;
    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    dim3 grid(tiles_n * tiles_m), block((TN / WN) * (TM / WM) * 64);
    hipLaunchKernelGGL((gemm_kernel<TN, TM, WN, WM, BK, BITS, GS, OUT, STAGES>), grid, block, 0,
                       stream, a, tiles_n, tiles_m, 8, SplitArgs{});
    return hipGetLastError();
}

template <int TN, int TM, int WN, int WM, int BK, int BITS, int GS, int OUT, int STAGES>
hipError_t launch_split_cfg(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                            hipStream_t stream)
{
    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    constexpr int U = GS ? GS / BK : 1;  // K tiles per split unit
    if (a.K % BK != 0 || p.splits < 2 || a.K / BK / U < p.splits || p.tiles != (int64_t)tiles_n * tiles_m ||
        p.tile_elems != (int64_t)TN * TM)
        return hipErrorInvalidValue;  // the plan does not fit this configuration
    dim3 grid(tiles_n * tiles_m * p.splits), block((TN / WN) * (TM / WM) * 64);
    hipLaunchKernelGGL((gemm_kernel<TN, TM, WN, WM, BK, BITS, GS, OUT, STAGES, true>), grid, block, 0,
                       stream, a, tiles_n, tiles_m, 8, SplitArgs{part, cnt, p.splits});
    return hipGetLastError();
}

// Compute units of the current device (workgroups that run at once when
// each takes a whole compute unit).
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

int64_t rounds(int64_t M, int64_t N, int TM, int TN)
{
    const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    const int64_t cu = compute_units();
    return (tiles + cu - 1) / cu;
}

// Tile shape by M (measured on MI355X over the N=10240 / N=2560 operator
// shapes).  M <= 128: 64 channels x 32 / 64 / 128 tokens with deep K tiles;
// M <= 256: 64-channel x 128-token tiles with a deep copy ring
// (latency-bound: more copies in flight).  Up to 1024 tokens: 160-channel
// tiles (int8 above 512 tokens: 8 waves of 160 x 64 over 256 tokens, 10%
// faster than 128 tokens at M = 768..1024).  Larger M: a big tile, chosen by
// how many whole rounds of workgroups over the compute units it needs times
// its measured time per tile: 320 x 256 (8 waves of 160 x 64), or 256 x 256
// (8 waves of 128 x 64, about 0.8x the time per tile on HBM-cold operands).
// int4 follows the same rule since its widening costs five VALU operations per
// 8 codes (it used to favour a 4-wave 128 x 128 layout that widens each
// weight fragment once for 4 token blocks).
template <int BITS, int OUT>
hipError_t launch_bits(const ProductArgs &a, hipStream_t stream)
{
    // Few tokens: the weights stream through once, so each K tile is deep
    // (128 bytes of a weight row, 256 for packed int4) to read whole cache
    // lines per row and halve the tiles, and with them the per-tile barrier
    // and wait latency that bounds a workgroup's rate here.
    constexpr int BKS = BITS == 8 ? 128 : 256, STS = BITS == 8 ? 4 : 3;
    if (a.M <= 128 && a.K % BKS == 0) {  // whole deep tiles only
        if (a.M <= 32)
            return launch_cfg<64, 32, 32, 32, BKS, BITS, 0, OUT, STS>(a, stream);
        if (a.M <= 64)
            return launch_cfg<64, 64, 32, 64, BKS, BITS, 0, OUT, STS>(a, stream);
        return launch_cfg<64, 128, 32, 64, BKS, BITS, 0, OUT, STS>(a, stream);
    }
    if (a.M <= 256)
        return launch_cfg<64, 128, 32, 64, 64, BITS, 0, OUT, 8>(a, stream);
    if (BITS == 8 && a.M > 512 && a.M <= 1024)
        return launch_cfg<160, 256, 160, 64, 64, BITS, 0, OUT, 4>(a, stream);
    if (a.M <= 1024)
        return launch_cfg<160, 128, 160, 32, 64, BITS, 0, OUT, 4>(a, stream);
    const int64_t r320 = rounds(a.M, a.N, 256, 320), r256 = rounds(a.M, a.N, 256, 256);
    if (100 * r320 <= 80 * r256)
        return launch_cfg<320, 256, 160, 64, 64, BITS, 0, OUT, 4>(a, stream);
    return launch_cfg<256, 256, 128, 64, 64, BITS, 0, OUT, 4>(a, stream);
}

// Per group (operands swapped; a wave owns 32 tokens of WN channels).
template <int BITS, int GS, int OUT>
hipError_t launch_group(const ProductArgs &a, hipStream_t stream)
{
    if (a.M <= 768)
        return launch_cfg<64, 128, 64, 32, 64, BITS, GS, OUT, 6>(a, stream);
    if (a.M <= 1536)
        return launch_cfg<128, 128, 64, 32, 64, BITS, GS, OUT, 4>(a, stream);
    if (a.M <= 3072)
        return launch_cfg<160, 128, 160, 32, 64, BITS, GS, OUT, 3>(a, stream);
    return launch_cfg<320, 128, 160, 32, 64, BITS, GS, OUT, 4>(a, stream);  // fewer re-reads of X
}

template <int GS, int OUT>
hipError_t launch_group_bits(const ProductArgs &a, hipStream_t stream)
{
    return a.bits == 8 ? launch_group<8, GS, OUT>(a, stream) : launch_group<4, GS, OUT>(a, stream);
}

// Split-K tiles for few tokens: 64 channels x 32 / 64 / 128 tokens; per
// channel with the deep K tiles of the unsplit few-token product, per group
// with 64-deep tiles (whole groups per split).
constexpr int kSplitTN = 64;
constexpr int split_tm(int64_t M) { return M <= 32 ? 32 : M <= 64 ? 64 : 128; }
constexpr int split_bk(int bits, int group_size) { return group_size ? 64 : bits == 8 ? 128 : 256; }

template <int BITS, int GS, int OUT>
hipError_t launch_split_bits(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream)
{
    if constexpr (GS == 0) {
        constexpr int BKS = BITS == 8 ? 128 : 256, STS = BITS == 8 ? 4 : 3;
        if (a.M <= 32)
            return launch_split_cfg<kSplitTN, 32, 32, 32, BKS, BITS, 0, OUT, STS>(a, p, part, cnt, stream);
        if (a.M <= 64)
            return launch_split_cfg<kSplitTN, 64, 32, 64, BKS, BITS, 0, OUT, STS>(a, p, part, cnt, stream);
        return launch_split_cfg<kSplitTN, 128, 32, 64, BKS, BITS, 0, OUT, STS>(a, p, part, cnt, stream);
    } else {
        if (a.M <= 32)
            return launch_split_cfg<kSplitTN, 32, 64, 32, 64, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
        if (a.M <= 64)
            return launch_split_cfg<kSplitTN, 64, 64, 32, 64, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
        return launch_split_cfg<kSplitTN, 128, 64, 32, 64, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
    }
}

template <int OUT>
hipError_t launch_split_kind(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream)
{
    const bool b8 = a.bits == 8;
    switch (a.group_size) {
    case 0:
        return b8 ? launch_split_bits<8, 0, OUT>(a, p, part, cnt, stream)
                  : launch_split_bits<4, 0, OUT>(a, p, part, cnt, stream);
    case 64:
        return b8 ? launch_split_bits<8, 64, OUT>(a, p, part, cnt, stream)
                  : launch_split_bits<4, 64, OUT>(a, p, part, cnt, stream);
    default:
        return b8 ? launch_split_bits<8, 128, OUT>(a, p, part, cnt, stream)
                  : launch_split_bits<4, 128, OUT>(a, p, part, cnt, stream);
    }
}

}  // namespace

// When to split, from measurements of the whole layer on MI355X (N = 10240,
// K = 2560 per channel; N = 2560, K = 10240 per group; 16 to 256 tokens):
//   * per group (up to 256 tokens): the unsplit few-token kernel takes
//     35-70 us; split into about one workgroup per compute unit, the
//     matrix-core tiles take 26-42 us;
//   * int4 per channel (up to 64 tokens): about two workgroups per compute
//     unit, 12-14% faster;
//   * int8 per channel: never faster -- the deep-K tiles already stream the
//     weights at the rate the split reaches, and the partial sums' round trip
//     through memory costs more than the extra workgroups gain.
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int bits, int group_size)
{
    SplitPlan p{1, 0, 0};
    const int bk = split_bk(bits, group_size);
    const int64_t max_m = group_size ? 256 : bits == 4 ? 64 : 0;
    if (M < 1 || M > max_m || N < 1 || K < bk || K % bk != 0)
        return p;
    const int TM = split_tm(M);
    const int64_t tiles = ((N + kSplitTN - 1) / kSplitTN) * ((M + TM - 1) / TM);
    const int64_t units = K / bk / (group_size ? group_size / bk : 1);
    const int64_t target = (group_size ? 1 : 2) * (int64_t)compute_units();
    int64_t S = (target + tiles / 2) / tiles;  // nearest
    S = S < 8 ? S : 8;
    S = S < units ? S : units;
    if (S < 2)
        return p;
    p.splits = (int)S;
    p.tiles = tiles;
    p.tile_elems = (int64_t)kSplitTN * TM;
    return p;
}

hipError_t launch_gemm_split(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream)
{
    switch (a.out_kind) {
    case OUT_F16: return launch_split_kind<OUT_F16>(a, p, part, cnt, stream);
    case OUT_BF16: return launch_split_kind<OUT_BF16>(a, p, part, cnt, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int OUT>
hipError_t launch_kind(const ProductArgs &a, hipStream_t stream)
{
    if (a.group_size == 64)
        return launch_group_bits<64, OUT>(a, stream);
    if (a.group_size == 128)
        return launch_group_bits<128, OUT>(a, stream);
    if (a.bits == 8)
        return launch_bits<8, OUT>(a, stream);
    return launch_bits<4, OUT>(a, stream);
}

hipError_t launch_gemm(const ProductArgs &a, hipStream_t stream)
{
    if (a.M <= 256 && a.group_size != 0)
        return launch_gemm_skinny(a, stream);
    switch (a.out_kind) {
    case OUT_F16: return launch_kind<OUT_F16>(a, stream);
    case OUT_BF16: return launch_kind<OUT_BF16>(a, stream);
    default: return launch_kind<OUT_I32>(a, stream);
    }
}

}  // namespace cider
