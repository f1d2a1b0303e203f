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
// SPLIT (per group only): workgroup blockIdx.x computes split z = blockIdx.x / tiles of tile
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
        // Each split stores its partials, waits for them to complete, meets
        // the workgroup barrier, and thread 0 counts the split in with an
        // agent-scope acquire-release read-modify-write: the release part
        // publishes every wave's stores (ordered before it by the barrier)
        // to the whole device, and in the last split to count in the
        // acquire part, followed by the barrier, orders every wave's loads
        // of the other splits' partials after their stores (the AMDGPU
        // memory model, gfx942 / gfx950 code sequences: release = write back
        // the XCD's L2 and wait, acquire = invalidate the caches).  The
        // partials themselves are relaxed agent-scope atomics.  The
        // partials are added in split order, so the sum does not depend on
        // which split was last.
        static_assert(SCALED, "split products are per group and dequantize");
        constexpr int TILE = TM * TN;
        typedef unsigned long long u64;
        uint32_t *mine = static_cast<uint32_t *>(sp.part) + (int64_t)pid * sp.splits * TILE +
                         wave * (64 * FN * FM * 16) + lane * 4;
        auto slot = [&](int zz, int i, int j, int q) {
            return reinterpret_cast<u64 *>(mine + (int64_t)zz * TILE + ((i * FM + j) * 4 + q) * 256);
        };
        auto quarter = [&](int i, int j, int q) -> i32x4 {
            return i32x4{__float_as_int(facc[i][j][4 * q]), __float_as_int(facc[i][j][4 * q + 1]),
                         __float_as_int(facc[i][j][4 * q + 2]), __float_as_int(facc[i][j][4 * q + 3])};
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
            *flag = __hip_atomic_fetch_add(sp.cnt + pid, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
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
                            const float f = __int_as_float(v[i][j][q][e]);
                            facc[i][j][4 * q + e] = first_split ? f : facc[i][j][4 * q + e] + f;
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
                    packed.x = pack2<OUT>(y[0], y[1]);
                    packed.y = pack2<OUT>(y[2], y[3]);
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

// Persistent per-channel product for many tokens (int8 or packed int4
// weights).  Same arithmetic as gemm_kernel per channel; what differs is how
// the operands reach the matrix cores:
//   * K tiles are 128 bytes of every token row (a whole 128-byte line; packed
//     int4 weight rows give 64 bytes).  Copying 64-byte halves of lines, each
//     line is requested from L2 twice; measured on this chip, a compute unit
//     then pulls about 17.6 bytes per clock from L2 against 25.6 with whole
//     lines, and the 320 x 256 tile needs about 29 per clock to keep its
//     matrix cores busy.
//   * The LDS ring has two stages of one 128-deep K tile each (72 KB for
//     int8).  Tile kt is computed from stage kt & 1 in four 32-deep steps;
//     the one barrier per K tile sits before the fourth step, after which the
//     stage of tile kt is refilled with tile kt + 2 while the fourth step's
//     MFMAs run.
//   * One workgroup per compute unit walks several output tiles.  The first
//     K tile of its next output tile is copied during the current tile's last
//     K tile and epilogue; the epilogue stages its fp16 rows in the other
//     (idle) stage of the ring.
//   * Outputs leave through range-checked buffer stores (out-of-range rows
//     and channels are dropped by the hardware), so every wave issues the same
//     number of memory instructions and the in-order vmcnt waits count
//     exactly.
// Needs K % 128 == 0 and K >= 256 (two K tiles).

// Channel blocks (of 32) per staging pass: the largest power of two up to
// fn whose 32 rows (cb * 64 bytes + 16 of padding each) fit in wreg bytes.
constexpr int cb_for(int fn, int wreg)
{
    int cb = 1;
    while (cb * 2 <= fn && 32 * (cb * 2 * 64 + 16) <= wreg)
        cb *= 2;
    return cb;
}

template <int TN, int TM, int WN, int WM, int BITS, int OUT>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_wide_kernel(ProductArgs args, int tiles_n,
                                                                               int tiles_m, int group_m)
{
    constexpr int BK = 128;
    constexpr int NWN = TN / WN, NWM = TM / WM, NW = NWN * NWM;
    constexpr int FN = WN / 32, FM = WM / 32;
    constexpr int XROW = BK, WROW = BITS == 8 ? BK : BK / 2;
    constexpr int XBYTES = TM * XROW, WBYTES = TN * WROW;
    constexpr int STAGE = XBYTES + WBYTES;
    constexpr int XB = XBYTES / 1024, WB = WBYTES / 1024, TB = XB + WB;
    constexpr int D = (XB + NW - 1) / NW + (WB + NW - 1) / NW;  // copies per wave per K tile
    static_assert(XBYTES % 1024 == 0 && WBYTES % 1024 == 0, "tiles of whole 1 KB blocks");
    static_assert(WN % 32 == 0 && WM % 32 == 0 && TN % WN == 0 && TM % WM == 0, "whole 32 x 32 blocks per wave");
    constexpr bool USUM = BITS == 4;  // unsigned int4 codes, corrected by the token sums
    // epilogue: each wave stages CB channel blocks of 32 tokens at a time in
    // its share of the idle stage (rows of 64 * CB bytes padded by 16)
    constexpr int WREG = STAGE / NW;
    constexpr int CB = cb_for(FN, WREG);
    constexpr int NPASS = (FN + CB - 1) / CB;
    static_assert((FN % CB & (FN % CB - 1)) == 0, "the last pass is a power of two wide too");
    constexpr int ROWB = CB * 64 + 16;
    // fp16 stores per wave per output tile: per token block and pass, 32 rows
    // of cb * 64 bytes in 16-byte pieces; int32: one 16-byte store per
    // (token block, channel block, quarter)
    constexpr int STORES = OUT == OUT_I32 ? FM * FN * 4 : FM * FN * 2;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) float s_sw[OUT != OUT_I32 ? TN : 4];
    __shared__ __attribute__((aligned(16))) float s_st[OUT != OUT_I32 ? TM : 4];

    const int64_t M = args.M, N = args.N, K = args.K;
    const int KT = (int)(K / BK);
    const int tiles = tiles_n * tiles_m;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWN, wm = wave / NWN;
    const int frow = lane & 31, fhalf = lane >> 5;
    const uint32_t wld = (uint32_t)(BITS == 8 ? K : K / 2);
    const i32x4 rX = make_rsrc(args.xq, (uint32_t)(M * K));
    const i32x4 rW = make_rsrc(args.wq, (uint32_t)(N * (int64_t)wld));

    // Copies: each wave takes DX consecutive 1 KB blocks of the token tile and
    // DW of the weight tile (clamped repeats of the last block when they do not
    // split evenly, so every wave issues D = DX + DW copies per K tile).  A
    // block holds 1024 / ROW consecutive rows; lane l takes row l / (ROW / 16)
    // of it and LDS slot l % (ROW / 16), which receives global chunk
    // slot ^ swizzle(row).  For these row lengths the swizzle depends on the
    // block only through its parity (128-byte rows) or not at all (64-byte
    // rows), so two per-lane offsets serve every block.
    constexpr int DX = (XB + NW - 1) / NW, DW = (WB + NW - 1) / NW;
    constexpr int CX = XROW / 16, CW = WROW / 16;
    constexpr int RX = 1024 / XROW, RW = 1024 / WROW;  // rows per block
    uint32_t xlane[2], wlane[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int rx = par * RX + lane / CX;
        xlane[par] = (uint32_t)((lane / CX) * K) + (((lane % CX) ^ swz8<BK>(rx)) << 4);
        const int rw = par * RW + lane / CW;
        wlane[par] = (uint32_t)((lane / CW) * (int64_t)wld) +
                     (((lane % CW) ^ (BITS == 8 ? swz8<BK>(rw) : swz4<BK>(rw))) << 4);
    }
    const uint32_t smem_lds = lds_address(smem);
    const uint32_t xstep = (uint32_t)(RX * K), wstep = (uint32_t)(RW * (int64_t)wld);
    // Copy j (0 <= j < D: DX token blocks, then DW weight blocks) of K tile kt
    // of the output tile at (m0, n0) into `stage`.
    auto copy_one = [&](int j, int stage, int64_t m0, int64_t n0, int kt) {
        const uint32_t lds = smem_lds + stage * STAGE;
        if (j < DX) {
            const int b = min(wave * DX + j, XB - 1);  // wavefront-uniform
            const uint32_t u = (uint32_t)(m0 * K) + (uint32_t)kt * XROW + (uint32_t)b * xstep;
            dma16(rX, lds + b * 1024, xlane[b & 1] + u);
        } else {
            const int b = min(wave * DW + (j - DX), WB - 1);
            const uint32_t u = (uint32_t)(n0 * (int64_t)wld) + (uint32_t)kt * WROW + (uint32_t)b * wstep;
            dma16(rW, lds + XBYTES + b * 1024, wlane[b & 1] + u);
        }
    };
    // all D copies of a K tile (the empty asm keeps the compiler from
    // precomputing one register per copy: two per-lane offsets and uniform
    // terms are enough)
    auto copy_tile = [&](int stage, int64_t m0, int64_t n0, int kt) {
        asm volatile("" : "+v"(xlane[0]), "+v"(xlane[1]), "+v"(wlane[0]), "+v"(wlane[1]));
#pragma unroll
        for (int j = 0; j < D; ++j)
            copy_one(j, stage, m0, n0, kt);
    };

    struct Frags {
        i32x4 a[FN];
        uint2 ap[BITS == 4 ? FN : 1];
        i32x4 b[FM];
    };
    constexpr int LOADS = FN + FM;
    // Fragment addresses.  Rows of a fragment are 32 consecutive rows starting
    // at a multiple of 32, so their swizzle depends on the lane only: one base
    // address per operand, and fragment k lies 32 rows further (an immediate
    // offset).  Step ks flips address bits (ks << 5) (int8 rows: chunk
    // 2 ks + half) or (ks << 4) (packed int4 rows: chunk ks), inside the row.
    const uint32_t abase = BITS == 8 ? (uint32_t)(XBYTES + (wn * WN + frow) * WROW + ((fhalf ^ swz8<BK>(frow)) << 4))
                                     : (uint32_t)(XBYTES + (wn * WN + frow) * WROW + (swz4<BK>(frow) << 4) + fhalf * 8);
    const uint32_t bbase = (uint32_t)((wm * WM + frow) * XROW + ((fhalf ^ swz8<BK>(frow)) << 4));
    auto load_frags = [&](Frags &f, int stage, int ks) {
        const uint32_t a = (abase + (uint32_t)(stage * STAGE)) ^ (uint32_t)(ks << (BITS == 8 ? 5 : 4));
        const uint32_t b = (bbase + (uint32_t)(stage * STAGE)) ^ (uint32_t)(ks << 5);
#pragma unroll
        for (int k = 0; k < FN; ++k) {
            if constexpr (BITS == 8)
                f.a[k] = *reinterpret_cast<const i32x4 *>(smem + a + k * 32 * WROW);
            else
                f.ap[k] = *reinterpret_cast<const uint2 *>(smem + a + k * 32 * WROW);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
            f.b[j] = *reinterpret_cast<const i32x4 *>(smem + b + j * 32 * XROW);
    };
    auto widen = [&](Frags &f, int i) {
        if constexpr (BITS == 4) {
            uint32_t d0, d1, d2, d3;
            unpack8u(f.ap[i].x, d0, d1);
            unpack8u(f.ap[i].y, d2, d3);
            f.a[i] = i32x4{(int)d0, (int)d1, (int)d2, (int)d3};
        }
    };

    i32x16 acc[FN][FM];
    int xs[USUM ? FM : 1];
    // One 32-deep step: the D copies of the K tile at (cm0, cn0, ckt) into
    // `cstage` first when `copies` (a short burst; the other wave of the SIMD
    // keeps its matrix core busy meanwhile), then the MFMAs on `cur` with the
    // fragment reads of the next step (into `nxt`, from stage `lstage`, step
    // `lks`) spread between them.  (Raising the wave priority around the MFMAs
    // helped an LDS-resident copy of this loop but made the product 2-3%
    // slower; issuing the copies one per MFMA instead of in a burst was no
    // faster.)
    auto step = [&](Frags &cur, Frags &nxt, bool reads, int lstage, int lks, bool copies, int cstage,
                    int64_t cm0, int64_t cn0, int ckt) {
        if (copies)
            copy_tile(cstage, cm0, cn0, ckt);
        __builtin_amdgcn_sched_barrier(0);
        if (reads)
            load_frags(nxt, lstage, lks);
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
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
        }
        constexpr int PER = (FN * FM) / LOADS > 0 ? (FN * FM) / LOADS : 1;
#pragma unroll
        for (int k = 0; k < LOADS; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // then MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // The dequant scales of an output tile go into registers early (loaded
    // before the previous tile's epilogue, so their latency hides) and into
    // LDS before its own epilogue.  Indices are clamped into range; values
    // past the edge are never used.
    constexpr int NSC = OUT != OUT_I32 ? (TN + TM + NW * 64 - 1) / (NW * 64) : 0;
    static_assert(NSC + STORES + D < 64, "vmcnt range");
    float scv[NSC > 0 ? NSC : 1], scn[NSC > 0 ? NSC : 1];
    auto load_scales = [&](float (&dst)[NSC > 0 ? NSC : 1], int64_t m0, int64_t n0) {
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int q = (int)threadIdx.x + i * NW * 64;
            const float *src = q < TN ? args.s_w + min(n0 + q, N - 1)
                                      : args.s_tok + min(m0 + min(q - TN, TM - 1), M - 1);
            dst[i] = *src;
        }
    };

    int t = blockIdx.x;
    if (t >= tiles)
        return;
    int tn, tm;
    tile_coords(t, tiles_n, tiles_m, group_m, tn, tm);
    int g = 0;  // K tiles this workgroup has consumed: K tile kt of the current output tile is in stage (g + kt) & 1
    load_scales(scv, (int64_t)tm * TM, (int64_t)tn * TN);
    copy_tile(0, (int64_t)tm * TM, (int64_t)tn * TN, 0);
    copy_tile(1, (int64_t)tm * TM, (int64_t)tn * TN, 1);
    wait_vmcnt<D>();  // K tile 0 has landed
    for (;;) {
        const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;
        const int tnext = t + (int)gridDim.x;
        const bool has_next = tnext < tiles;  // workgroup-uniform
        int tn2 = 0, tm2 = 0;
        if (has_next)
            tile_coords(tnext, tiles_n, tiles_m, group_m, tn2, tm2);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = i32x16{};
#pragma unroll
        for (int j = 0; j < (USUM ? FM : 1); ++j)
            xs[j] = 0;
        __builtin_amdgcn_s_barrier();  // K tile 0 of this output tile is in, in every wave's view
        __builtin_amdgcn_sched_barrier(0);
        Frags f0, f1;
        load_frags(f0, g & 1, 0);
        for (int kt = 0; kt < KT; ++kt) {
            const int cs = (g + kt) & 1, ns = cs ^ 1;
            const bool last = kt == KT - 1;
            step(f0, f1, true, cs, 1, false, 0, 0, 0, 0);
            step(f1, f0, true, cs, 2, false, 0, 0, 0, 0);
            step(f0, f1, true, cs, 3, false, 0, 0, 0, 0);
            // Every wave is done reading stage cs.  Before the barrier: K tile
            // kt + 1 has landed (it is the newest copy in flight, except in the
            // last K tile, where the next output tile's first K tile may follow).
            wait_lgkm0();
            if (!last)
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // refill stage cs: K tile kt + 2, or the next output tile's first
            const bool own = kt + 2 < KT, nxt_tile = kt + 2 == KT && has_next;
            step(f1, f0, !last, ns, 0, own || nxt_tile, cs, own ? m0 : (int64_t)tm2 * TM,
                 own ? n0 : (int64_t)tn2 * TN, own ? kt + 2 : 0);
        }
        const int es = (g + KT - 1) & 1;  // the stage of the last K tile: idle now
        g += KT;
        // the next output tile's scales (after its first K tile's copies, before
        // this tile's stores: the wait for those copies below counts them)
        load_scales(scn, (int64_t)tm2 * TM, (int64_t)tn2 * TN);

        if constexpr (USUM) {
            // both halves of each token's K: sum q x = sum u x - 8 sum x
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int s8 = 8 * (xs[j] + __shfl_xor(xs[j], 32, 64));
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[i][j][e] -= s8;
            }
        }

        // Epilogue.  Block (i, j) gives the lane token m = wm*WM + 32j + lane%32
        // and, for q = 0..3, channels nb .. nb+3, nb = wn*WN + 32i + 8q + 4*(lane/32).
        // (The lane index is re-derived behind an empty asm so that no
        // epilogue address is computed once before the tile loop and kept
        // live through it.)
        int elane = (int)threadIdx.x & 63;
        asm volatile("" : "+v"(elane));
        const int frow = elane & 31, fhalf = elane >> 5;
        if constexpr (OUT == OUT_I32) {
            const uint64_t ybase = reinterpret_cast<uint64_t>(args.out) + (uint64_t)m0 * (uint64_t)N * 4u;
            const auto ry = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ybase), (short)0,
                                                              (int)(min((int64_t)TM, M - m0) * N * 4), 0x00020000);
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int r = wm * WM + j * 32 + frow;
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t nb = n0 + wn * WN + i * 32 + q * 8 + fhalf * 4;
                        const uint32_t off = nb < N ? (uint32_t)(((int64_t)r * N + nb) * 4) : 0x80000000u;
                        const i32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                         acc[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, 0);
                    }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                const int q = (int)threadIdx.x + i * NW * 64;
                if (q < TN)
                    s_sw[q] = scv[i];
                else if (q < TN + TM)
                    s_st[q - TN] = scv[i];
            }
            __syncthreads();  // scales in LDS; every wave is done with stage es
            const uint64_t ybase = reinterpret_cast<uint64_t>(args.out) + (uint64_t)m0 * (uint64_t)N * 2u;
            const auto ry = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ybase), (short)0,
                                                              (int)(min((int64_t)TM, M - m0) * N * 2), 0x00020000);
            // Dequantize every block to packed 16-bit values first (half the
            // registers of the int32 sums), channel block by channel block so
            // each block's scales are read once for both token blocks.
            float st[FM];
#pragma unroll
            for (int j = 0; j < FM; ++j)
                st[j] = s_st[wm * WM + j * 32 + frow];
            uint2 pk[FN][FM][4];
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 sw = *reinterpret_cast<const f32x4 *>(&s_sw[wn * WN + i * 32 + q * 8 + fhalf * 4]);
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        float y[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            y[e] = (float)acc[i][j][4 * q + e] * st[j] * sw[e];
                        pk[i][j][q].x = pack2<OUT>(y[0], y[1]);
                        pk[i][j][q].y = pack2<OUT>(y[2], y[3]);
                    }
                }
            const uint32_t rowbytes = (uint32_t)N * 2u;
            const int nvalid = (int)min((int64_t)TN, N - n0);  // channels of this tile inside N
            // Then 32 token rows at a time through this wave's share of the idle
            // stage (rows of CB channel blocks, padded by 16 bytes so the 32 rows
            // a write touches fall in distinct bank groups), leaving as 16-byte
            // pieces, consecutive lanes along a token row.
            uint8_t *ob = smem + es * STAGE + wave * WREG;
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int p = 0; p < NPASS; ++p) {
                    const int i0 = p * CB;
                    const int ncb = min(CB, FN - i0);  // compile-time after unrolling
#pragma unroll
                    for (int ii = 0; ii < CB; ++ii)
                        if (ii < ncb)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                *reinterpret_cast<uint2 *>(ob + frow * ROWB + (ii * 32 + q * 8 + fhalf * 4) * 2) =
                                    pk[i0 + ii][j][q];
                    // ncb * 4 pieces of 16 bytes per row (a power of two up to 16):
                    // lane l takes piece l % cpr of rows l / cpr + it * 64 / cpr
                    const int cpr = ncb * 4;
                    const int lr = elane / cpr, lc = elane % cpr;
                    const int nc = wn * WN + i0 * 32 + lc * 8;  // channel within the tile
                    const uint32_t base = nc < nvalid ? (uint32_t)(wm * WM + j * 32 + lr) * rowbytes +
                                                            (uint32_t)(n0 + nc) * 2u
                                                      : 0x80000000u;  // past the buffer: dropped
                    const uint8_t *src = ob + lr * ROWB + lc * 16;
#pragma unroll
                    for (int it = 0; it < 32 * cpr / 64; ++it) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(src + it * (64 / cpr) * ROWB);
                        __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ry,
                                                               base + (uint32_t)(it * (64 / cpr)) * rowbytes, 0,
                                                               2 /* non-temporal */);
                    }
                }
        }
        if (!has_next)
            break;
        // every wave is done with stage es and with the scales; refill es with
        // K tile 1 of the next output tile and wait for its K tile 0 (copied
        // before this tile's stores)
        __syncthreads();
        t = tnext;
        tn = tn2;
        tm = tm2;
#pragma unroll
        for (int i = 0; i < NSC; ++i)
            scv[i] = scn[i];
        copy_tile(es, (int64_t)tm * TM, (int64_t)tn * TN, 1);  // es == (g + 1) & 1
        // after K tile 0: the scale loads, the stores, K tile 1's copies
        wait_vmcnt<NSC + STORES + D>();
    }
    wait_vmcnt<0>();
}

// Persistent per-group product for many tokens (int8 or packed int4
// weights, groups of 64 / 128 along K; a wave owns one or two 32-token blocks
// of WN channels): the copy path of gemm_wide_kernel
// (128-byte K tiles, one workgroup per compute unit walking output tiles,
// copies streaming across tiles) with the operands of the
// per-group gemm_kernel (tokens are operand A, so a lane's outputs belong to
// one channel per 32-channel block and need one group scale each).  The
// channel scales of a K tile's groups travel with it into the ring.
//
// What differs is where the group scale-accumulate runs: the int32 sums of
// block i of a closed group are converted and scaled into the fp32 sums
// (16 conversions and 16 FMAs per lane) just before block i's first MFMA of
// the next group, so the vector ALU works on one block while the matrix core
// works on the previous one, instead of all blocks in one burst after the
// group's last MFMA.  The last group of an output tile is scaled before its
// epilogue.  Outputs leave as 2-byte range-checked buffer stores, consecutive
// lanes along a token row.
//
// The ring has STG stages of one K tile each; K tile kt + STG is copied into
// the stage of K tile kt once every wave is done reading it, so STG - 1 K
// tiles are in flight while one is computed.  Small output tiles (little
// matrix work per K tile) need the deeper rings to cover the copy latency.
// Every K tile issues its copies even when no K tile is left to fetch (a
// repeat of the current one, never read), so the in-order copy counts stay
// fixed.  Needs K % 128 == 0, K >= 128 * STG, fp16 / bf16 output.
template <int TN, int TM, int WN, int WM, int BITS, int GS, int OUT, int STG>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_group_wide_kernel(ProductArgs args, int tiles_n,
                                                                                     int tiles_m, int group_m)
{
    constexpr int BK = 128;
    constexpr int NWN = TN / WN, NWM = TM / WM, NW = NWN * NWM;
    constexpr int FN = WN / 32;  // 32-channel blocks per wave
    constexpr int FM = WM / 32;  // 32-token blocks per wave
    static_assert(WM % 32 == 0 && WN % 32 == 0 && TN % WN == 0 && TM % WM == 0, "whole 32 x 32 blocks per wave");
    static_assert(OUT != OUT_I32, "the int32 hook takes gemm_kernel");
    constexpr int XROW = BK, WROW = BITS == 8 ? BK : BK / 2;
    constexpr int XBYTES = TM * XROW, WBYTES = TN * WROW;
    constexpr int GPT = BK / GS;  // groups per K tile
    constexpr int SPG = GS / 32;  // 32-deep steps per group
    constexpr int SBYTES = (GPT * TN * 4 + 1023) / 1024 * 1024;
    constexpr int STAGE = XBYTES + WBYTES + SBYTES;
    constexpr int XB = XBYTES / 1024, WB = WBYTES / 1024, SB = GPT * TN / 64;
    constexpr int DX = (XB + NW - 1) / NW, DW = (WB + NW - 1) / NW, DS = (SB + NW - 1) / NW;
    constexpr int D = DX + DW + DS;  // copies per wave per K tile
    static_assert(XBYTES % 1024 == 0 && WBYTES % 1024 == 0 && TN % 64 == 0, "whole copy blocks");
    constexpr int STORES = FN * FM * 16;  // 2-byte output stores per wave per output tile
    constexpr int NSC = (TM + NW * 64 - 1) / (NW * 64);

    static_assert(STG >= 2, "at least double buffering");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STG * STAGE];
    __shared__ __attribute__((aligned(16))) float s_st[TM];

    const int64_t M = args.M, N = args.N, K = args.K;
    const int KT = (int)(K / BK);
    const int G = (int)(K / GS);
    const int tiles = tiles_n * tiles_m;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWN, wm = wave / NWN;
    const int frow = lane & 31, fhalf = lane >> 5;
    const uint32_t wld = (uint32_t)(BITS == 8 ? K : K / 2);
    const i32x4 rX = make_rsrc(args.xq, (uint32_t)(M * K));
    const i32x4 rW = make_rsrc(args.wq, (uint32_t)(N * (int64_t)wld));
    const i32x4 rS = make_rsrc(args.s_w, (uint32_t)(N * G * 4));

    // Copies, as in gemm_wide_kernel; scale block sb (0 .. SB-1) holds the
    // tile's channels 64 (sb % (TN/64)) .. +63 of its group sb / (TN/64):
    // lane l copies s_w[n0 + 64 (sb % (TN/64)) + l, g0 + sb / (TN/64)] (past N:
    // out of range, reads 0).
    constexpr int CX = XROW / 16, CW = WROW / 16;
    constexpr int RX = 1024 / XROW, RW = 1024 / WROW;
    uint32_t xlane[2], wlane[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int rx = par * RX + lane / CX;
        xlane[par] = (uint32_t)((lane / CX) * K) + (((lane % CX) ^ swz8<BK>(rx)) << 4);
        const int rw = par * RW + lane / CW;
        wlane[par] = (uint32_t)((lane / CW) * (int64_t)wld) +
                     (((lane % CW) ^ (BITS == 8 ? swz8<BK>(rw) : swz4<BK>(rw))) << 4);
    }
    uint32_t slane = (uint32_t)lane * (uint32_t)G * 4u;
    const uint32_t smem_lds = lds_address(smem);
    const uint32_t xstep = (uint32_t)(RX * K), wstep = (uint32_t)(RW * (int64_t)wld);
    auto copy_tile = [&](int stage, int64_t m0, int64_t n0, int kt) {
        asm volatile("" : "+v"(xlane[0]), "+v"(xlane[1]), "+v"(wlane[0]), "+v"(wlane[1]), "+v"(slane));
        const uint32_t lds = smem_lds + stage * STAGE;
        const uint32_t xo = (uint32_t)(m0 * K) + (uint32_t)kt * XROW;
#pragma unroll
        for (int j = 0; j < DX; ++j) {
            const int b = min(wave * DX + j, XB - 1);  // wavefront-uniform
            dma16(rX, lds + b * 1024, xlane[b & 1] + xo + (uint32_t)b * xstep);
        }
        const uint32_t wo = (uint32_t)(n0 * (int64_t)wld) + (uint32_t)kt * WROW;
#pragma unroll
        for (int j = 0; j < DW; ++j) {
            const int b = min(wave * DW + j, WB - 1);
            dma16(rW, lds + XBYTES + b * 1024, wlane[b & 1] + wo + (uint32_t)b * wstep);
        }
#pragma unroll
        for (int j = 0; j < DS; ++j) {
            const int sb = min(wave * DS + j, SB - 1);
            const int gi = sb / (TN / 64), cb = sb % (TN / 64);
            const uint32_t so = (uint32_t)((n0 + cb * 64) * G + (int64_t)kt * GPT + gi) * 4u;
            dma4(rS, lds + XBYTES + WBYTES + sb * 256, slane + so);
        }
    };

    // Fragments: operand A = the wave's FM blocks of 32 token rows, operand
    // B = its FN 32-channel blocks (packed int4 bytes until widened).
    struct Frags {
        i32x4 x[FM];
        i32x4 w[FN];
        uint2 wp[BITS == 4 ? FN : 1];
    };
    const uint32_t xbase = (uint32_t)((wm * WM + frow) * XROW + ((fhalf ^ swz8<BK>(frow)) << 4));
    const uint32_t wbase = BITS == 8 ? (uint32_t)(XBYTES + (wn * WN + frow) * WROW + ((fhalf ^ swz8<BK>(frow)) << 4))
                                     : (uint32_t)(XBYTES + (wn * WN + frow) * WROW + (swz4<BK>(frow) << 4) + fhalf * 8);
    auto load_frags = [&](Frags &f, int stage, int ks) {
        const uint32_t a = (xbase + (uint32_t)(stage * STAGE)) ^ (uint32_t)(ks << 5);
        const uint32_t b = (wbase + (uint32_t)(stage * STAGE)) ^ (uint32_t)(ks << (BITS == 8 ? 5 : 4));
#pragma unroll
        for (int j = 0; j < FM; ++j)
            f.x[j] = *reinterpret_cast<const i32x4 *>(smem + a + j * 32 * XROW);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            if constexpr (BITS == 8)
                f.w[i] = *reinterpret_cast<const i32x4 *>(smem + b + i * 32 * WROW);
            else
                f.wp[i] = *reinterpret_cast<const uint2 *>(smem + b + i * 32 * WROW);
        }
    };
    // channel scales of the wave's blocks for group gi of the K tile in `stage`
    auto load_scales_lds = [&](float (&sw)[FN], int stage, int gi) {
        const float *ss = reinterpret_cast<const float *>(smem + stage * STAGE + XBYTES + WBYTES) + gi * TN;
#pragma unroll
        for (int i = 0; i < FN; ++i)
            sw[i] = ss[wn * WN + i * 32 + frow];
    };

    i32x16 acc[FN][FM];
    float facc[FN][FM][16];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
            acc[i][j] = i32x16{};
    // One 32-deep step.  first: the step opens a group: block i of the group
    // that closed before it is scaled into facc with the scales `sw` right
    // before block i's first MFMA (which starts from zero) overwrites its
    // sums.  (The first group of an output tile finds the previous tile's
    // already-scaled sums, or zeros, with scales 0.)
    auto step = [&](auto first, Frags &cur, Frags &nxt, bool reads, int lstage, int lks,
                    const float (&sw)[FN], bool copies, int cstage, int64_t cm0, int64_t cn0, int ckt) {
        if (copies)
            copy_tile(cstage, cm0, cn0, ckt);
        __builtin_amdgcn_sched_barrier(0);
        if (reads)
            load_frags(nxt, lstage, lks);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                if constexpr (decltype(first)::value) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        facc[i][j][e] += (float)acc[i][j][e] * sw[i];
                }
                if constexpr (BITS == 4) {
                    if (j == 0) {
                        uint32_t d0, d1, d2, d3;
                        unpack8(cur.wp[i].x, d0, d1);
                        unpack8(cur.wp[i].y, d2, d3);
                        cur.w[i] = i32x4{(int)d0, (int)d1, (int)d2, (int)d3};
                    }
                }
                if constexpr (decltype(first)::value) {
                    // Block (i, j)'s MFMA must follow its scaling: otherwise the
                    // compiler may run the new group's MFMAs first and keep both
                    // groups' sums live (twice the registers).  The weight
                    // fragment passes through an empty asm that takes the scaled
                    // sums as inputs.
                    const float(&f)[16] = facc[i][j];
                    asm volatile(""
                                 : "+v"(cur.w[i])
                                 : "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(f[4]), "v"(f[5]), "v"(f[6]),
                                   "v"(f[7]), "v"(f[8]), "v"(f[9]), "v"(f[10]), "v"(f[11]), "v"(f[12]),
                                   "v"(f[13]), "v"(f[14]), "v"(f[15]));
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.x[j], cur.w[i], i32x16{}, 0, 0, 0);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.x[j], cur.w[i], acc[i][j], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    auto load_tok_scales = [&](float (&dst)[NSC], int64_t m0) {
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int q = (int)threadIdx.x + i * NW * 64;
            dst[i] = args.s_tok[min(m0 + min(q, TM - 1), M - 1)];
        }
    };
    float scv[NSC], scn[NSC];

    int t = blockIdx.x;
    if (t >= tiles)
        return;
    int tn, tm;
    tile_coords(t, tiles_n, tiles_m, group_m, tn, tm);
    int cs = 0;  // the stage of the K tile being computed (K tile 0 of the first output tile: 0)
    load_tok_scales(scv, (int64_t)tm * TM);
#pragma unroll
    for (int j = 0; j < STG; ++j)
        copy_tile(j, (int64_t)tm * TM, (int64_t)tn * TN, j);
    wait_vmcnt<D * (STG - 1)>();  // K tile 0 has landed
    for (;;) {
        const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;
        const int tnext = t + (int)gridDim.x;
        const bool has_next = tnext < tiles;  // workgroup-uniform
        int tn2 = 0, tm2 = 0;
        if (has_next)
            tile_coords(tnext, tiles_n, tiles_m, group_m, tn2, tm2);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    facc[i][j][e] = 0.f;
        __builtin_amdgcn_s_barrier();  // K tile 0 of this output tile is in, in every wave's view
        __builtin_amdgcn_sched_barrier(0);
        Frags f0, f1;
        load_frags(f0, cs, 0);
        // scales of the group waiting to be scaled (read from the ring before
        // the barrier after which its stage may be refilled)
        float swp[FN];
#pragma unroll
        for (int i = 0; i < FN; ++i)
            swp[i] = 0.f;
        for (int kt = 0; kt < KT; ++kt) {
            const int ns = cs + 1 == STG ? 0 : cs + 1;
            const bool last = kt == KT - 1;
            step(Flag<true>{}, f0, f1, true, cs, 1, swp, false, 0, 0, 0, 0);
            step(Flag<false>{}, f1, f0, true, cs, 2, swp, false, 0, 0, 0, 0);
            if constexpr (GPT == 2) {
                float swa[FN];  // the K tile's first group, closed after step 1
                load_scales_lds(swa, cs, 0);
                step(Flag<true>{}, f0, f1, true, cs, 3, swa, false, 0, 0, 0, 0);
            } else {
                step(Flag<false>{}, f0, f1, true, cs, 3, swp, false, 0, 0, 0, 0);
            }
            // the group closing at this K tile's end is scaled in the next K
            // tile (or before the epilogue)
            load_scales_lds(swp, cs, GPT - 1);
            wait_lgkm0();
            if (!last)
                wait_vmcnt<D * (STG - 2)>();  // K tile kt + 1 has landed
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // refill stage cs with the next K tile not yet copied: K tile
            // kt + STG of this output tile, or K tile kt + STG - KT of the
            // next; past the last output tile, a repeat of K tile kt
            const bool own = kt + STG < KT;
            const bool nxt_tile = !own && has_next;
            step(Flag<false>{}, f1, f0, !last, ns, 0, swp, true, cs,
                 nxt_tile ? (int64_t)tm2 * TM : m0, nxt_tile ? (int64_t)tn2 * TN : n0,
                 own ? kt + STG : nxt_tile ? kt + STG - KT : kt);
            cs = ns;
        }
        load_tok_scales(scn, (int64_t)tm2 * TM);  // after the next tile's first copies
        // the last group
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    facc[i][j][e] += (float)acc[i][j][e] * swp[i];

        // Epilogue: y = s_tok[m] * facc.  Block (i, j): channel n = wn*WN +
        // 32i + lane%32, tokens wm*WM + 32j + 8q + 4*(lane/32) + e for element
        // 4q + e.
#pragma unroll
        for (int i = 0; i < NSC; ++i) {
            const int q = (int)threadIdx.x + i * NW * 64;
            if (q < TM)
                s_st[q] = scv[i];
        }
        __syncthreads();  // token scales in LDS (the previous tile's readers are past its barrier)
        int elane = (int)threadIdx.x & 63;
        asm volatile("" : "+v"(elane));
        const int er = elane & 31, eh = elane >> 5;
        const uint32_t rowbytes = (uint32_t)N * 2u;
        const uint64_t ybase = reinterpret_cast<uint64_t>(args.out) + (uint64_t)m0 * (uint64_t)N * 2u;
        const auto ry = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ybase), (short)0,
                                                          (int)(min((int64_t)TM, M - m0) * N * 2), 0x00020000);
        const int nvalid = (int)min((int64_t)TN, N - n0);
        f32x4 stv[FM][4];
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                stv[j][q] = *reinterpret_cast<const f32x4 *>(&s_st[wm * WM + j * 32 + q * 8 + eh * 4]);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int nc = wn * WN + i * 32 + er;
            const uint32_t base = nc < nvalid ? (uint32_t)(wm * WM + eh * 4) * rowbytes + (uint32_t)(n0 + nc) * 2u
                                              : 0x80000000u;  // past the buffer: dropped
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float y = stv[j][q][e] * facc[i][j][4 * q + e];
                        __builtin_amdgcn_raw_buffer_store_b16(
                            out_bits<OUT>(y), ry, base + (uint32_t)(j * 32 + q * 8 + e) * rowbytes, 0, 2);
                    }
        }
        if (!has_next)
            break;
        __syncthreads();  // every wave is done reading the token scales
        t = tnext;
        tn = tn2;
        tm = tm2;
#pragma unroll
        for (int i = 0; i < NSC; ++i)
            scv[i] = scn[i];
        // the next tile's K tile 0 is older than its K tiles 1 .. STG - 1, the
        // token scale loads and this tile's stores
        constexpr int AFTER0 = D * (STG - 1) + NSC + STORES;
        wait_vmcnt<(AFTER0 < 63 ? AFTER0 : 63)>();
    }
    wait_vmcnt<0>();
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

template <int TN, int TM, int WN, int WM, int BITS, int OUT>
hipError_t launch_wide(const ProductArgs &a, hipStream_t stream)
{

    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    const int tiles = tiles_n * tiles_m;
    int grid = compute_units();
    if (grid > tiles)
        grid = tiles;
    hipLaunchKernelGGL((gemm_wide_kernel<TN, TM, WN, WM, BITS, OUT>), dim3(grid), dim3((TN / WN) * (TM / WM) * 64),
                       0, stream, a, tiles_n, tiles_m, 8);
    return hipGetLastError();
}

template <int TN, int TM, int WN, int WM, int BITS, int GS, int OUT, int STG>
hipError_t launch_group_wide(const ProductArgs &a, hipStream_t stream)
{
    if (a.K % 128 != 0 || a.K < 128 * STG)  // whole K tiles, the ring filled by one output tile
        return hipErrorInvalidValue;
    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    const int tiles = tiles_n * tiles_m;
    int grid = compute_units();
    if (grid > tiles)
        grid = tiles;
    hipLaunchKernelGGL((gemm_group_wide_kernel<TN, TM, WN, WM, BITS, GS, OUT, STG>), dim3(grid),
                       dim3((TN / WN) * (TM / WM) * 64), 0, stream, a, tiles_n, tiles_m, 8);
    return hipGetLastError();
}

int64_t rounds(int64_t M, int64_t N, int TM, int TN)
{
    const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    const int64_t cu = compute_units();
    return (tiles + cu - 1) / cu;
}

// Tile shape by M (measured on MI355X over the N=10240 / N=2560 operator
// shapes).  M <= 128: 64 channels x 32 / 64 / 128 tokens with deep K tiles;
// up to 192 the 64 x 64 tiles repeated over M, up to 384 128 x 128 deep-K
// tiles, int8 up to 576 128 x 192, up to 768 128 x 256 and up to 1024
// 160 x 256 deep-K tiles (each where it makes about one round).
// Past that, with whole 128-byte K tiles (at least two) and outputs
// addressable with 32-bit offsets, the persistent kernel with the smallest
// output tile whose tiles all run at once, one per compute unit: 160 x 128
// (4 waves of 160 x 32), 160 x 256 (4 waves of 160 x 64), else 256 x 256
// (8 waves of 128 x 64), 320 x 256 (8 waves of 160 x 64) or, with int8
// weights, 192 x 256 (8 waves of 96 x 64) over several rounds, by rounds
// times time per tile (M = 1280 / 1536 / 2560 / 3072, int8:
// 256 x 256 45.0 -> 41.2, 46.3 -> 44.3, 85.0 -> 74.2, 89.6 -> 79.9 us; at
// M = 2048, 3584, 4096 and 6144 it needs one more round than 320 x 256 and
// loses, 53.5 -> 73.6 us at 2048).  A second round costs a whole
// tile time again (at N = 10240, K = 2560, int8 / int4: 160 x 128 tiles take
// 23.6-26.0 / 21.1-22.6 us for M = 192..512 in one round and 45.1 / 40.2 us
// at M = 768 in two; 160 x 256: 33.7 / 32.9 us at M = 768; the earlier
// 64 x 128 and 160 x 128 / 160 x 256 tiles of gemm_kernel with 64-byte K
// tiles: 26.6-34.2 / 26.1-37.7 us over M = 192..768, 36.7 / 41.9 us at
// M = 1024, where 160 x 256 takes 35.7 / 34.6 us).
// Otherwise (K not a multiple of 128): 64 x 128 tiles with a deep copy ring
// up to 256 tokens (latency-bound: more copies in flight), 160-channel tiles
// up to 1024 (int8 above 512 tokens: 8 waves of 160 x 64 over 256 tokens),
// then 320 x 256 or 256 x 256 by how many whole rounds of workgroups over the
// compute units each needs times its measured time per tile (256 x 256 takes
// about 0.8x the time per tile on HBM-cold operands).
template <int BITS, int OUT>
hipError_t launch_bits(const ProductArgs &a, hipStream_t stream)
{
    // Few tokens: the weights stream through once, so each K tile is deep
    // (128 bytes of a weight row, 256 for packed int4) to read whole cache
    // lines per row and halve the tiles, and with them the per-tile barrier
    // and wait latency that bounds a workgroup's rate here.
    // One wave per 32 x 32 block (4 waves at 64 tokens, 8 at 128): at
    // N = 10240, K = 2560, M = 64 the product takes 11.4 / 11.1 us (int8 /
    // int4) against 12.4 / 13.3 with waves of 32 x 64; deeper rings and
    // 128-channel tiles measured no faster.
    constexpr int BKS = BITS == 8 ? 128 : 256, STS = BITS == 8 ? 4 : 3;
    if (a.M <= 128 && a.K % BKS == 0) {  // whole deep tiles only
        if (a.M <= 32)
            return launch_cfg<64, 32, 32, 32, BKS, BITS, 0, OUT, STS>(a, stream);
        if (a.M <= 64)
            return launch_cfg<64, 64, 32, 32, BKS, BITS, 0, OUT, STS>(a, stream);
        return launch_cfg<64, 128, 32, 32, BKS, BITS, 0, OUT, STS>(a, stream);
    }
    // 129..512 tokens, deep K tiles of the same kernel where they make about
    // one round of workgroups, which the one-round persistent tiles (160 x
    // 128, 4 waves) do not beat here: they leave compute units idle or run
    // too few waves per unit.  At N = 10240, K = 2560 (product, us; persistent
    // 160 x 128 in brackets): 64 x 64 tiles repeated over M, M = 160 / 192:
    // int8 15.1 / 16.0 (23.3 / 23.7), int4 14.7 / 14.4 (22.0 / 22.4), and
    // 16.5 against 14.0 for the 64 x 128 tiles at 128 tokens; 128 x 128 tiles
    // of 8 waves of 64 x 32, M = 256 / 320 / 384: int8 17.2 / 16.4 / 17.3
    // (21.7 for 96 x 128 at 256; 23.6 / 25.7 at 320 / 384), int4 M = 256 /
    // 288 / 384: 19.6 / 19.5 / 19.8 (20.5 / 22.2 / 23.2); int8 128 x 192 tiles
    // of 12 waves, M = 448 / 512 / 576: 21.4 / 21.9 / 23.1 (23.8 / 25.8 /
    // 31.7; 128 x 128: 29.7 / 31.3 at 448 / 512, two rounds); int8 128 x 256
    // tiles of 8 waves of 64 x 64, M = 640 / 768: 24.5 / 26.0 (persistent
    // 160 x 256: 31.2 / 32.8; at 896 / 1024 they need two rounds, 42.3 /
    // 45.6 against 33.5 / 35.9).
    // (Each only where its workgroups fit that round: the 64 x 64 tiles two
    // per compute unit, the others one; wider layers keep the persistent
    // tiles below.)  int8 160 x 256 tiles of 8 waves of 160 x 32, M = 896 /
    // 1024: 30.5 / 31.9 (persistent 160 x 256 of 4 waves: 32.5 / 35.1).
    const int64_t ncu = compute_units();
    auto fits = [&](int64_t tn, int64_t tm, int64_t per_cu) {
        return (a.N + tn - 1) / tn * ((a.M + tm - 1) / tm) <= per_cu * ncu;
    };
    // int4, 513..768 tokens: 128 x 256 tiles of 8 waves of 64 x 64 with
    // 128-value K tiles (64-byte packed rows), M = 640 / 768: 26.7 / 28.2 us
    // against 34.6 / 34.9 for the persistent 160 x 256 tiles (at 448 / 512:
    // 26.3 / 26.4 against 22.7 / 23.5 for 160 x 128).
    if constexpr (BITS == 4) {
        if (a.M > 512 && a.M <= 768 && a.K % 128 == 0 && fits(128, 256, 1))
            return launch_cfg<128, 256, 64, 64, 128, BITS, 0, OUT, 3>(a, stream);
    }
    if (a.K % BKS == 0) {
        if (a.M <= 192 && fits(64, 64, 2))
            return launch_cfg<64, 64, 32, 32, BKS, BITS, 0, OUT, STS>(a, stream);
        if (a.M <= 384 && fits(128, 128, 1))
            return launch_cfg<128, 128, 64, 32, BKS, BITS, 0, OUT, STS>(a, stream);
        if constexpr (BITS == 8) {
            if (a.M <= 576 && fits(128, 192, 1))
                return launch_cfg<128, 192, 64, 32, BKS, BITS, 0, OUT, 3>(a, stream);
            if (a.M <= 768 && fits(128, 256, 1))
                return launch_cfg<128, 256, 64, 64, BKS, BITS, 0, OUT, 3>(a, stream);
            if (a.M <= 1024 && fits(160, 256, 1))
                return launch_cfg<160, 256, 160, 32, BKS, BITS, 0, OUT, 3>(a, stream);
        }
    }
    if (a.K % 128 == 0 && a.K >= 256 && 256 * a.N * 4 < (int64_t(1) << 31)) {
        const int64_t cu = compute_units();
        auto one_round = [&](int64_t tn, int64_t tm) { return (a.N + tn - 1) / tn * ((a.M + tm - 1) / tm) <= cu; };
        if (one_round(160, 128))
            return launch_wide<160, 128, 160, 32, BITS, OUT>(a, stream);
        if (one_round(160, 256))
            return launch_wide<160, 256, 160, 64, BITS, OUT>(a, stream);
        // several rounds: rounds times the time per tile, relative to a
        // 320 x 256 tile: 256 x 256 about 0.88, and (int8) 192 x 256 (8 waves
        // of 96 x 64) about 0.81 -- more time per unit of work, but whole
        // rounds where the larger tiles leave the last round half empty (the
        // 4096 x 6144 x 4096 product of the decoder stack's QKV projection:
        // 192 x 256 100.3 us against 109.1 for 256 x 256 and 127.0 for
        // 320 x 256; at 4096 x 10240 x 2560 it needs 4 rounds and takes
        // 130.0 against 102.1 us)
        const int64_t t320 = 100 * rounds(a.M, a.N, 256, 320), t256 = 88 * rounds(a.M, a.N, 256, 256);
        if constexpr (BITS == 8) {
            const int64_t t192 = 81 * rounds(a.M, a.N, 256, 192);
            if (t192 < t256 && t192 < t320)
                return launch_wide<192, 256, 96, 64, BITS, OUT>(a, stream);
        }
        if (t256 < t320)
            return launch_wide<256, 256, 128, 64, BITS, OUT>(a, stream);
        return launch_wide<320, 256, 160, 64, BITS, OUT>(a, stream);
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
//
// Past the few-token range, the persistent kernel: of the tiles whose
// output tiles all run at once, one per compute unit, the one with the
// fewest rows per K tile (64 x 96, 64 x 128, 128 x 96, 128 x 128, 192 x 128,
// 256 x 128 channels x tokens, each with a ring deep enough to cover the copy
// latency of its little matrix work per K tile).  96-token tiles: M = 1024
// int8 gs64 / gs128 88.3 / 81.2 -> 79.7 / 74.7 us (128 x 96 against
// 128 x 128); M = 300..512 gs128 50.0-52.2 -> 47.2-47.6 us (64 x 96 against
// 64 x 128), gs64 unchanged.  Measured time per
// output tile at N = 2560, K = 10240 (one tile per compute unit, int8 gs64 /
// gs128): 60 / 52, 88 / 81, 128 / 110 and 148 / 126 us for 64 to 256
// channels; a second round of tiles costs a whole tile time again, so the
// narrowest tile that needs one round wins (M = 512 and 768: 80.6 / 71.0 us
// before, 60.5 / 52.5 after; M = 1024: 96.0 / 99.7 -> 88.4 / 81.4 us; M =
// 2048: 141.2 / 138.4 -> 128.1 / 109.8 us; M = 3072: 180.6 / 164.3 ->
// 148.0 / 125.9 us).  Past one round of 256-channel tiles: groups of 128
// take the 320-channel persistent kernel (M = 4096: int8 176.7 -> 153.3 us,
// int4 209.1 -> 199.9 us on one box); groups of 64 the 320 x 128 tiles of
// gemm_kernel, which the persistent kernel did not beat there (187.2 ->
// 187.6 us; int4 238 -> 249 us): there the scale-accumulate's two vector
// operations per output and group bound both kernels.
template <int BITS, int GS, int OUT>
hipError_t launch_group(const ProductArgs &a, hipStream_t stream)
{
    if constexpr (OUT != OUT_I32) {
        // whole 128-byte K tiles; 128-token output tiles addressable with
        // 32-bit offsets
        if (a.K % 128 == 0 && 128 * a.N * 2 < (int64_t(1) << 31)) {
            const int64_t cu = compute_units(), tiles_m = (a.M + 127) / 128;
            auto one_round = [&](int64_t tn) { return (a.N + tn - 1) / tn * tiles_m <= cu; };
            auto one_round96 = [&](int64_t tn) { return (a.N + tn - 1) / tn * ((a.M + 95) / 96) <= cu; };
            if (a.K >= 512) {  // the deepest ring below holds 4 K tiles
                // candidates in order of rows per K tile (TN + TM)
                if (one_round96(64))
                    return launch_group_wide<64, 96, 64, 32, BITS, GS, OUT, 4>(a, stream);
                if (one_round(64))
                    return launch_group_wide<64, 128, 64, 32, BITS, GS, OUT, 4>(a, stream);
                if (one_round96(128))
                    return launch_group_wide<128, 96, 64, 32, BITS, GS, OUT, 3>(a, stream);
                if (one_round(128))
                    return launch_group_wide<128, 128, 64, 32, BITS, GS, OUT, 3>(a, stream);
                if (one_round(192))
                    return launch_group_wide<192, 128, 64, 32, BITS, GS, OUT, 3>(a, stream);
                if (one_round(256))
                    return launch_group_wide<256, 128, 128, 32, BITS, GS, OUT, 3>(a, stream);
            }
            // int4 weights past that: 192 x 256 tiles of 8 waves of 96 x 64, so
            // every widened weight fragment feeds two token blocks (half the
            // widening per MFMA): gs64 / gs128 M = 4096 246.3 / 204.8 ->
            // 210.4 / 177.8 us, M = 8192 481.8 / 397.5 -> 412.7 / 349.0 us
            // (int8: within +-3 %, kept).  Below one round of them they lose
            // to the small one-round tiles (M = 2048 gs64 142.4 against
            // 207.5 us).
            if constexpr (BITS == 4) {
                if (a.M > 3072 && a.K >= 256 && 256 * a.N * 2 < (int64_t(1) << 31))
                    return launch_group_wide<192, 256, 96, 64, BITS, GS, OUT, 2>(a, stream);
            }
            if (GS == 128 && a.M > 3072 && a.K >= 256)
                return launch_group_wide<320, 128, 160, 32, BITS, GS, OUT, 2>(a, stream);
        }
    }
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

// Split-K tiles for few tokens (per group only): 64 channels x 32 / 64 / 128
// tokens with 64-deep K tiles (whole groups per split).  Up to 64 tokens the
// tile's channels are split over two waves (32 x 32 each; 4 waves at 64
// tokens): whole layers at N = 2560, K = 10240 gs64, M = 16 / 32 / 64 take
// 23.8 / 24.3 / 26.7 us against 27.6 / 28.3 / 29.6 with one wave per 32
// tokens; at 128 tokens that split measured slower (37.4 against 35.0 us).
constexpr int kSplitTN = 64;
constexpr int kSplitBK = 64;
constexpr int split_tm(int64_t M) { return M <= 32 ? 32 : M <= 64 ? 64 : 128; }

template <int BITS, int GS, int OUT>
hipError_t launch_split_bits(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream)
{
    if (a.M <= 32)
        return launch_split_cfg<kSplitTN, 32, 32, 32, kSplitBK, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
    if (a.M <= 64)
        return launch_split_cfg<kSplitTN, 64, 32, 32, kSplitBK, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
    return launch_split_cfg<kSplitTN, 128, 64, 32, kSplitBK, BITS, GS, OUT, 6>(a, p, part, cnt, stream);
}

template <int OUT>
hipError_t launch_split_kind(const ProductArgs &a, const SplitPlan &p, void *part, uint32_t *cnt,
                             hipStream_t stream)
{
    const bool b8 = a.bits == 8;
    switch (a.group_size) {
    case 0:
        return hipErrorInvalidValue;  // per-channel products are never split
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
//   * per channel (int8 and int4): never faster -- the deep-K tiles already
//     stream the weights at the rate the split reaches, and the partial sums'
//     round trip plus the acquire-release handoff (an L2 write-back per
//     workgroup) cost more than the extra workgroups gain (int4, 16 / 32 / 64
//     tokens: 20.6 / 21.6 / 24.7 us split, 15.0 / 15.2 / 17.0 us unsplit).
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int bits, int group_size)
{
    SplitPlan p{1, 0, 0};
    if (group_size == 0 || M < 1 || M > 256 || N < 1 || K < group_size || K % group_size != 0)
        return p;
    // Up to 32 tokens the few-token kernel is faster unsplit (int8 gs64,
    // N = 2560, K = 10240, M = 16: 12.9 us against about 20 us split).
    ProductArgs fa{};
    fa.M = M;
    fa.N = N;
    fa.K = K;
    fa.bits = bits;
    fa.group_size = group_size;
    fa.out_kind = OUT_F16;
    if (few_supported(fa))
        return p;
    const int TM = split_tm(M);
    const int64_t tiles = ((N + kSplitTN - 1) / kSplitTN) * ((M + TM - 1) / TM);
    const int64_t units = K / group_size;
    const int64_t target = compute_units();
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

// Unsplit products (the product entry points, and linear calls without the
// split workspace).  Per group from 33 to 256 tokens the few-token kernel's
// 32-token tiles, repeated over M (the weights re-read from L2), beat the
// skinny kernel everywhere measured and the persistent per-group tiles up to
// 192 int8-weight tokens (N = 2560, K = 10240, product alone; skinny / few /
// persistent): int8 gs64 M = 64: 34.0 / 27.7 / 59.9 us, M = 128: 60.6 /
// 40.1 / 60.2, M = 192: 61.4 / 52.3 / 60.5, M = 256: 89.2 / 65.6 / 60.4;
// gs128 M = 128: 52.0 / 36.2 / 46.8, M = 256: 76.3 / 59.3 / 47.1; int4 gs64
// M = 128: 58.8 / 34.4 / 81.3, M = 256: - / 54.9 / 81.4; int4 gs128 M = 256:
// 74.9 / 46.3 / 70.0; int4 gs64 / gs128 M = 320: - / 73.1 / 81.1 and
// - / 61.5 / 69.7, M = 384: - / 83.8 / 81.2 and - / 70.6 / 69.5.  So int4
// takes the few-token tiles up to 320 tokens, int8 up to 192, and int8
// 193..256 tokens the persistent tiles (whole 128-byte K tiles, deep enough
// for their ring); the skinny kernel keeps the shapes none of them takes and
// the per-group int32 hook.
hipError_t launch_gemm(const ProductArgs &a, hipStream_t stream)
{
    if (few_supported(a))
        return launch_gemm_few(a, stream);
    if (a.group_size != 0 && a.M <= (a.bits == 4 ? 320 : 192) && few_shape_ok(a))
        return launch_gemm_few(a, stream);
    if (a.M <= 256 && a.group_size != 0) {
        if (a.bits == 8 && a.out_kind != OUT_I32 && a.K % 128 == 0 && a.K >= 512 &&
            128 * a.N * 2 < (int64_t(1) << 31))
            return a.out_kind == OUT_F16 ? launch_kind<OUT_F16>(a, stream) : launch_kind<OUT_BF16>(a, stream);
        return launch_gemm_skinny(a, stream);
    }
    switch (a.out_kind) {
    case OUT_F16: return launch_kind<OUT_F16>(a, stream);
    case OUT_BF16: return launch_kind<OUT_BF16>(a, stream);
    default: return launch_kind<OUT_I32>(a, stream);
    }
}

}  // namespace cider
