// INT8 matrix-core product for the fused quantized linear layer on gfx950.
//
// What it computes (Cider README, ossradar.top repo page, "Quantization"
// table and "Metal Kernel Pipeline"): acc[m, n] = sum_k xq[m, k] * q_w[n, k]
// in int32, then y = fp16(acc * s_tok[m] * s_w[n]) in the same kernel
// ("TensorOps matmul2d": dequantization applied in the store phase).  Per
// group of 64/128 along K ("W8A8 Quantization Granularity"): each group's
// int32 sum is scaled by s_w[n, g] and added into an fp32 accumulator.  W4A8
// ("Modes": Unpack -> TensorOps): packed nibbles are widened to int8 codes
// before the int8 product.
//
// Design for CDNA4 (the pages' M5 tiling is prior art only):
//   * v_mfma_i32_32x32x32_i8: 32x32 int32 block, 32-deep K per instruction
//     (the full-rate int8 shape on gfx950; the 16x16x64 form issues at about
//     half the rate).  The weight tile is the A operand and the activation
//     tile the B operand, so each lane holds runs of four consecutive output
//     channels n of one token m: the epilogue stores 8 contiguous bytes.
//   * Tiles of TN x TM outputs per workgroup, WN x WM per wavefront, K
//     staged BK at a time through LDS, double buffered: global loads of tile
//     k+1 are in flight while the matrix cores consume tile k; one barrier
//     per K tile.
//   * LDS rows of BK bytes in 16-byte chunks, chunk c of row r stored at
//     slot c ^ swz(r): the 16 rows a fragment read touches (same chunk) land
//     in distinct bank groups, and so do the row-major tile writes.
//   * W4A8: a 16-byte global chunk of packed nibbles becomes two 16-byte
//     int8 chunks in LDS, once per workgroup; every wavefront then reads
//     plain int8 fragments.
//   * Workgroup -> tile mapping: consecutive workgroup ids go to different
//     XCDs (round robin over 8), so ids are remapped to give every XCD a
//     contiguous run of tiles, walked in groups of m-panels, so the tiles
//     sharing an L2 also share weight and activation panels.
#include "cider_kernels.h"

namespace cider {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;

template <int BK>
__device__ __forceinline__ int lds_offset(int row, int chunk)
{
    constexpr int CPR = BK / 16;  // 16-byte chunks per row
    static_assert(CPR == 4 || CPR == 8, "BK must be 64 or 128");
    // Conflict-free for 16-byte reads of consecutive rows at one chunk,
    // whether LDS serves 8 lanes per 128 bytes or 16 lanes per 256 bytes.
    const int swz = (CPR == 8) ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) ^ (row >> 2)) & 3);
    return row * BK + ((chunk ^ swz) << 4);
}

// Widen 8 packed nibbles (k = 0..7 of a uint32, low nibble = even k) to 8
// int8 codes q = u - 8 in k order: two dwords.
__device__ __forceinline__ void unpack_nibbles(uint32_t v, uint32_t &d0, uint32_t &d1)
{
    const uint32_t lo = v & 0x0F0F0F0Fu;          // u0 u2 u4 u6
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;   // u1 u3 u5 u7
    // interleave to u0 u1 u2 u3 | u4 u5 u6 u7
    uint32_t a = (lo & 0xFFu) | ((hi & 0xFFu) << 8) | ((lo & 0xFF00u) << 8) | ((hi & 0xFF00u) << 16);
    uint32_t b = ((lo >> 16) & 0xFFu) | ((hi >> 8) & 0xFF00u) | (lo & 0xFF000000u) >> 8 |
                 (hi & 0xFF000000u);
    // u in [0, 15] -> u - 8 as a two's complement byte, without carries
    // between bytes: (u + 0x78) stays below 0x100; flipping bit 7 then
    // subtracts 0x80.
    d0 = (a + 0x78787878u) ^ 0x80808080u;
    d1 = (b + 0x78787878u) ^ 0x80808080u;
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

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    // Raw buffer, stride 0: byte offsets, loads at or past `bytes` return 0.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// One wavefront-wide asynchronous copy of 64 x 16 bytes from global memory
// straight into LDS: lane l's 16 bytes land at lds_block + 16 * l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *lds_block,
                                      uint32_t voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_block, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt untouched
}

template <int TN, int TM, int BK, int WN, int WM, int BITS, int GS, int OUT>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_kernel(
    ProductArgs args, int tiles_n, int tiles_m, int group_m)
{
    constexpr int NWN = TN / WN, NWM = TM / WM, NT = NWN * NWM * 64, NWAVES = NT / 64;
    constexpr int FN = WN / 32, FM = WM / 32;          // 32 x 32 blocks per wavefront
    constexpr int KSTEPS = BK / 32;                    // 32-deep matrix-core steps per tile
    constexpr int GSD = GS ? GS : 1;                   // divisor-safe group size
    constexpr int GSTEPS = GS ? GS / 32 : KSTEPS;      // k-steps per scaling group
    constexpr int GPT = GS ? BK / GSD : 1;             // groups per K tile
    static_assert(GS == 0 || BK % GS == 0, "a K tile holds whole groups");
    constexpr int CPR = BK / 16;                       // 16-byte chunks per int8 LDS row
    constexpr int WROWB = BITS == 8 ? BK : BK / 2;     // weight bytes per row per K tile
    constexpr int XBLK = TM * BK / 1024, WBLK = TN * WROWB / 1024;  // 1 KB copy blocks
    static_assert(XBLK >= 1 && WBLK >= 1, "tiles of at least 1 KB");
    constexpr int XPW = (XBLK + NWAVES - 1) / NWAVES, WPW = (WBLK + NWAVES - 1) / NWAVES;
    constexpr bool SCALED_GROUPS = GS != 0 && OUT == OUT_F16;
    constexpr int SPT = SCALED_GROUPS ? (GPT * TN + NT - 1) / NT : 1;  // scales per thread

    // Two stages per operand as distinct LDS objects, so the copies into
    // one stage and the fragment reads from the other are never confused.
    __shared__ __attribute__((aligned(1024))) uint8_t sX0[TM * BK];
    __shared__ __attribute__((aligned(1024))) uint8_t sX1[TM * BK];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[TN * WROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW1[TN * WROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sU[BITS == 4 ? TN * BK : 16];  // int4 -> int8
    __shared__ __attribute__((aligned(16))) float sS0[SCALED_GROUPS ? GPT * TN : 4];
    __shared__ __attribute__((aligned(16))) float sS1[SCALED_GROUPS ? GPT * TN : 4];

    const int64_t M = args.M, N = args.N, K = args.K;
    int tn, tm;
    tile_coords(blockIdx.x, tiles_n, tiles_m, group_m, tn, tm);
    const int64_t n0 = (int64_t)tn * TN, m0 = (int64_t)tm * TM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
    const int wn = wave % NWN, wm = wave / NWN;
    const int G = GS ? (int)(K / GSD) : 1;
    const uint32_t wld = (uint32_t)(BITS == 8 ? K : K / 2);

    const __amdgpu_buffer_rsrc_t rX = make_rsrc(args.xq, (uint32_t)(M * K));
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(args.wq, (uint32_t)(N * (int64_t)wld));

    // Per-lane source offsets of this wavefront's copy blocks.  LDS row r
    // slot s must hold global chunk s ^ swz(r) (int8 tiles); packed int4
    // tiles are copied unswizzled and widened by the unpack pass.
    uint32_t xoff[XPW], woff[WPW];
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
        const int b = wave + j * NWAVES;
        const int r = b * (1024 / BK) + lane / CPR, sl = lane % CPR;
        const int c = sl ^ (lds_offset<BK>(r, 0) - r * BK) / 16;
        xoff[j] = (uint32_t)((m0 + r) * K) + c * 16;
    }
#pragma unroll
    for (int j = 0; j < WPW; ++j) {
        const int b = wave + j * NWAVES;
        if constexpr (BITS == 8) {
            const int r = b * (1024 / BK) + lane / CPR, sl = lane % CPR;
            const int c = sl ^ (lds_offset<BK>(r, 0) - r * BK) / 16;
            woff[j] = (uint32_t)((n0 + r) * (int64_t)wld) + c * 16;
        } else {
            constexpr int CPRP = WROWB / 16;
            const int r = b * (1024 / WROWB) + lane / CPRP, c = lane % CPRP;
            woff[j] = (uint32_t)((n0 + r) * (int64_t)wld) + c * 16;
        }
    }

    auto issue_copies = [&](const uint8_t *dX, const uint8_t *dW, int kt) {
        const uint32_t kx = (uint32_t)kt * BK, kw = (uint32_t)kt * WROWB;
#pragma unroll
        for (int j = 0; j < XPW; ++j)
            if (XBLK % NWAVES == 0 || wave + j * NWAVES < XBLK)  // wavefront-uniform
                dma16(rX, dX + (wave + j * NWAVES) * 1024, xoff[j] + kx);
#pragma unroll
        for (int j = 0; j < WPW; ++j)
            if (WBLK % NWAVES == 0 || wave + j * NWAVES < WBLK)
                dma16(rW, dW + (wave + j * NWAVES) * 1024, woff[j] + kw);
    };

    float sreg[SPT];
    auto load_scales = [&](int kt) {
        if constexpr (SCALED_GROUPS) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int id = min(tid + i * NT, GPT * TN - 1);
                const int gi = id / TN, row = id % TN;
                const int64_t gr = min(n0 + row, N - 1);
                sreg[i] = args.s_w[gr * G + (int64_t)kt * GPT + gi];
            }
        }
    };
    auto store_scales = [&](float *dS) {
        if constexpr (SCALED_GROUPS) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int id = tid + i * NT;
                if (id < GPT * TN)
                    dS[id] = sreg[i];  // [gi][row]
            }
        }
    };
    // int4: widen the packed stage into sU (int8, swizzled like the others).
    auto unpack = [&](const uint8_t *dW) {
        if constexpr (BITS == 4) {
            constexpr int CPRP = WROWB / 16, TOTAL = TN * CPRP;
#pragma unroll
            for (int i = 0; i < (TOTAL + NT - 1) / NT; ++i) {
                const int id = tid + i * NT;
                if (TOTAL % NT == 0 || id < TOTAL) {
                    const int row = id / CPRP, c = id % CPRP;
                    const uint4 v = *reinterpret_cast<const uint4 *>(dW + row * WROWB + c * 16);
                    uint4 lo, hi;
                    unpack_nibbles(v.x, lo.x, lo.y);
                    unpack_nibbles(v.y, lo.z, lo.w);
                    unpack_nibbles(v.z, hi.x, hi.y);
                    unpack_nibbles(v.w, hi.z, hi.w);
                    *reinterpret_cast<uint4 *>(&sU[lds_offset<BK>(row, 2 * c)]) = lo;
                    *reinterpret_cast<uint4 *>(&sU[lds_offset<BK>(row, 2 * c + 1)]) = hi;
                }
            }
        }
    };

    i32x16 acc[GS == 0 ? FN : 1][GS == 0 ? FM : 1];
    f32x16 facc[SCALED_GROUPS ? FN : 1][SCALED_GROUPS ? FM : 1];
    if constexpr (GS == 0) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = i32x16{};
    }
    if constexpr (SCALED_GROUPS) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                facc[i][j] = f32x16{};
    }

    // v_mfma_i32_32x32x32_i8 operands: lane l holds row (l % 32) of a 32-row
    // block and 16 consecutive k of a 32-deep step (half l / 32).  Result:
    // lane l holds column l % 32 and, for q = 0..3, rows 8q + 4(l/32) + 0..3.
    const int frow = lane & 31, fhalf = lane >> 5;

    auto compute = [&](const uint8_t *tW, const uint8_t *tX, const float *tS, int kt) {
        if constexpr (GS == 0) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                i32x4 af[FN], bf[FM];
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    af[i] = *reinterpret_cast<const i32x4 *>(
                        tW + lds_offset<BK>(wn * WN + i * 32 + frow, s * 2 + fhalf));
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    bf[j] = *reinterpret_cast<const i32x4 *>(
                        tX + lds_offset<BK>(wm * WM + j * 32 + frow, s * 2 + fhalf));
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j],
                                                                          0, 0, 0);
            }
        } else {
#pragma unroll
            for (int gi = 0; gi < GPT; ++gi) {
                i32x4 af[GSTEPS][FN], bf[GSTEPS][FM];
#pragma unroll
                for (int s = 0; s < GSTEPS; ++s) {
                    const int ks = gi * GSTEPS + s;
#pragma unroll
                    for (int i = 0; i < FN; ++i)
                        af[s][i] = *reinterpret_cast<const i32x4 *>(
                            tW + lds_offset<BK>(wn * WN + i * 32 + frow, ks * 2 + fhalf));
#pragma unroll
                    for (int j = 0; j < FM; ++j)
                        bf[s][j] = *reinterpret_cast<const i32x4 *>(
                            tX + lds_offset<BK>(wm * WM + j * 32 + frow, ks * 2 + fhalf));
                }
                f32x4 sc[FN][4];
                if constexpr (SCALED_GROUPS) {
#pragma unroll
                    for (int i = 0; i < FN; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            sc[i][q] = *reinterpret_cast<const f32x4 *>(
                                &tS[gi * TN + wn * WN + i * 32 + q * 8 + fhalf * 4]);
                }
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        i32x16 t = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0][i], bf[0][j],
                                                                        i32x16{}, 0, 0, 0);
#pragma unroll
                        for (int s = 1; s < GSTEPS; ++s)
                            t = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s][i], bf[s][j], t, 0, 0, 0);
                        if constexpr (SCALED_GROUPS) {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    facc[i][j][4 * q + r] += (float)t[4 * q + r] * sc[i][q][r];
                        } else {
                            // raw per-group sums: out[(m * N + n) * G + g]
                            const int64_t m = m0 + wm * WM + j * 32 + frow;
                            if (m < M) {
                                int32_t *o = static_cast<int32_t *>(args.out);
                                const int64_t g = (int64_t)kt * GPT + gi;
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const int64_t n = n0 + wn * WN + i * 32 + q * 8 + fhalf * 4;
                                    if (n < N) {
#pragma unroll
                                        for (int r = 0; r < 4; ++r)
                                            o[(m * N + n + r) * G + g] = t[4 * q + r];
                                    }
                                }
                            }
                        }
                    }
            }
        }
    };

    const int KT = (int)(K / BK);
    issue_copies(sX0, sW0, 0);
    load_scales(0);
    store_scales(sS0);
    wait_vmem_all();
    __syncthreads();
    if constexpr (BITS == 4) {
        unpack(sW0);
        __syncthreads();
    }
    // One K tile per iteration: start the copies of tile kt+1 into the other
    // stage, run the matrix cores on this stage, then wait for the copies and
    // meet at a barrier.
    for (int kt = 0; kt < KT; ++kt) {
        const bool odd = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            issue_copies(odd ? sX0 : sX1, odd ? sW0 : sW1, kt + 1);
            load_scales(kt + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(BITS == 4 ? sU : (odd ? sW1 : sW0), odd ? sX1 : sX0, odd ? sS1 : sS0, kt);
        __builtin_amdgcn_sched_barrier(0);
        if (more)
            store_scales(odd ? sS0 : sS1);
        wait_vmem_all();
        __syncthreads();
        if constexpr (BITS == 4) {
            if (more) {
                unpack(odd ? sW0 : sW1);
                __syncthreads();
            }
        }
    }

    if constexpr (GS != 0 && OUT == OUT_I32)
        return;  // per-group sums were stored inside the loop

    // Epilogue: per block (i, j) the lane holds token m and, for q = 0..3,
    // output channels nb .. nb+3 with nb = block base + 8q + 4 * (lane / 32).
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int64_t m = m0 + wm * WM + j * 32 + frow;
        if (m >= M)
            continue;
        float st = 0.f;
        if constexpr (OUT == OUT_F16)
            st = args.s_tok[m];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t nb = n0 + wn * WN + i * 32 + q * 8 + fhalf * 4;
                if (nb >= N)
                    continue;
                if constexpr (OUT == OUT_I32) {
                    const i32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    *reinterpret_cast<i32x4 *>(static_cast<int32_t *>(args.out) + m * N + nb) = v;
                } else {
                    float y[4];
                    if constexpr (GS == 0) {
                        const f32x4 sw = *reinterpret_cast<const f32x4 *>(args.s_w + nb);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            y[r] = (float)acc[i][j][4 * q + r] * st * sw[r];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            y[r] = st * facc[i][j][4 * q + r];
                    }
                    uint2 packed;
                    packed.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[0]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[1]) << 16);
                    packed.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[2]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y[3]) << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(args.out) + m * N + nb) =
                        packed;
                }
            }
        }
    }
}

template <int TN, int TM, int BK, int WN, int WM, int BITS, int GS, int OUT>
hipError_t launch_cfg(const ProductArgs &a, hipStream_t stream)
{
    const int tiles_n = (int)((a.N + TN - 1) / TN);
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    const int group_m = 8;
    dim3 grid(tiles_n * tiles_m), block((TN / WN) * (TM / WM) * 64);
    hipLaunchKernelGGL((gemm_kernel<TN, TM, BK, WN, WM, BITS, GS, OUT>), grid, block, 0, stream,
                       a, tiles_n, tiles_m, group_m);
    return hipGetLastError();
}

// Tile shapes: (TN, TM, BK, WN, WM).
template <int BITS, int GS, int OUT>
hipError_t launch_mode(const ProductArgs &a, hipStream_t stream)
{
    // group_size 128 implies K % 128 == 0, so those always take 128-deep tiles.
    const bool bk128 = a.K % 128 == 0;
    if (a.M >= 512) {
        if constexpr (GS == 0) {
            if (bk128)
                return launch_cfg<256, 256, 128, 128, 128, BITS, GS, OUT>(a, stream);
            return launch_cfg<256, 256, 64, 128, 128, BITS, GS, OUT>(a, stream);
        } else if constexpr (GS == 128) {
            return launch_cfg<256, 128, 128, 64, 64, BITS, GS, OUT>(a, stream);
        } else {
            if (bk128)
                return launch_cfg<256, 128, 128, 64, 64, BITS, GS, OUT>(a, stream);
            return launch_cfg<256, 128, 64, 64, 64, BITS, GS, OUT>(a, stream);
        }
    }
    if constexpr (GS == 128) {
        return launch_cfg<64, 64, 128, 32, 32, BITS, GS, OUT>(a, stream);
    } else {
        if (bk128)
            return launch_cfg<64, 64, 128, 32, 32, BITS, GS, OUT>(a, stream);
        return launch_cfg<64, 64, 64, 32, 32, BITS, GS, OUT>(a, stream);
    }
}

}  // namespace

hipError_t launch_gemm(const ProductArgs &a, hipStream_t stream)
{
    if (a.group_size == 0)
        return launch_gemm_pc(a, stream);
    const bool f16 = a.out_kind == OUT_F16;
    if (a.bits == 8) {
        switch (a.group_size) {
        case 64: return f16 ? launch_mode<8, 64, OUT_F16>(a, stream) : launch_mode<8, 64, OUT_I32>(a, stream);
        case 128: return f16 ? launch_mode<8, 128, OUT_F16>(a, stream) : launch_mode<8, 128, OUT_I32>(a, stream);
        default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace cider
