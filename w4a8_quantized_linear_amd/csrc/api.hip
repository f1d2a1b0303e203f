// C ABI of the fused quantized linear layer (declared in include/cider.h).
//
// Host side only: argument checks (all before the first HIP call), the
// device check, the choice between the matrix-vector and the matrix-core
// kernel (Cider README, ossradar.top repo page, "Quick Start": seq_len > 1 ->
// INT8 GEMM, seq_len == 1 -> INT8 MV kernel), and the launches on the
// caller's stream.  No allocation, no synchronization.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "cider.h"
#include "cider_kernels.h"

namespace {

constexpr int64_t kMaxK = 133144;       // K * 127^2 < 2^31
constexpr int64_t kGemvMaxBytes = 65536;  // M * K int8 codes held in LDS (kernel limit)
constexpr int64_t kMaxOperandBytes = int64_t(1) << 31;
constexpr int64_t kDecodeMaxK = 32768;  // decode kernel: 16 activation chunks per thread, x [K] in LDS

std::atomic<int> g_path{0};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Bytes of the split product's partial sums (4-byte words per tile and
// split), and those plus the tile counters.
size_t split_part_bytes(const cider::SplitPlan &p)
{
    return round256((size_t)(p.tiles * p.splits * p.tile_elems) * 4u);
}
size_t split_bytes(const cider::SplitPlan &p)
{
    return split_part_bytes(p) + round256((size_t)p.tiles * sizeof(uint32_t));
}

// 1: usable gfx950 device current; 0: not.  Cached per device id.
int device_usable()
{
    const char *force = std::getenv("CIDER_FORCE_UNAVAILABLE");
    if (force && force[0] == '1')
        return 0;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 0;
    }
    static std::atomic<int> cache[64];  // 0 unknown, 1 usable, 2 not usable
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c)
            return c == 1;
    }
    hipDeviceProp_t prop;
    int ok = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
        ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    else
        (void)hipGetLastError();
    if (dev < 64)
        cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

cider_status from_hip(hipError_t e) { return e == hipSuccess ? CIDER_OK : CIDER_ERR_HIP; }

// Workspace of cider_linear_ex_noalloc: a device array of fixed size, one per
// GPU, kept for the life of the process.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
__device__ __align__(256) uint8_t scratch[CIDER_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's scratch address, or nullptr when it cannot be had.
void *scratch_address()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p)
        return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch_ptr[dev].store(addr, std::memory_order_release);
    return addr;
}

// Shape / mode checks shared by the product calls.
cider_status check_shape(int64_t M, int64_t N, int64_t K, int bits, int group_size)
{
    if (M < 0 || N < 0 || K <= 0)
        return CIDER_ERR_INVALID_ARG;
    if (bits != 8 && bits != 4)
        return CIDER_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return CIDER_ERR_INVALID_ARG;
    if (K % 64 != 0 || K > kMaxK || N % 64 != 0)
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    if (group_size && K % group_size != 0)
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    // The kernels address operands with 32-bit byte offsets (one tile past
    // the end included): each operand stays below 2 GiB.
    if ((M + 256) * K >= kMaxOperandBytes || (N + 256) * K >= kMaxOperandBytes)
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    return CIDER_OK;
}

enum Path { PATH_AUTO = 0, PATH_GEMV = 1, PATH_GEMM = 2 };

// Which kernel serves M tokens of K features; CIDER_ERR_UNSUPPORTED_SHAPE
// when the matrix-vector kernel is forced outside its range.  Automatic: the
// matrix-vector kernel (one pass over the weights, each token's dot products
// on the vector ALUs) where it measured faster than the matrix-core products
// on the operator shapes (N=10240 K=2560 and N=2560 K=10240, every mode,
// whole layer): where the few-token matrix-core kernel takes the product, up
// to 3 tokens per channel and 2 per group (per channel int8, M = 3 / 4:
// 8.9 / 10.8 us against 10.2 / 10.1; per group int8 gs64, M = 2 / 3: 11.3 /
// 15.6 against 15.0 / 15.1); elsewhere up to 8 int8-weight or 4 int4-weight
// tokens.
cider_status pick_path(int64_t M, int64_t N, int64_t K, int bits, int group_size, cider::OutKind kind,
                       int *path)
{
    const int forced = g_path.load(std::memory_order_relaxed);
    const bool gemv_ok = M <= 8 && M * K <= kGemvMaxBytes;
    cider::ProductArgs fa{};
    fa.M = M;
    fa.N = N;
    fa.K = K;
    fa.bits = bits;
    fa.group_size = group_size;
    fa.out_kind = kind;
    const int64_t gemv_max = cider::few_supported(fa) ? (group_size ? 2 : 3) : (bits == 4 ? 4 : 8);
    const bool gemv_auto = gemv_ok && M <= gemv_max;
    if (forced == PATH_GEMV) {
        if (!gemv_ok)
            return CIDER_ERR_UNSUPPORTED_SHAPE;
        *path = PATH_GEMV;
    } else if (forced == PATH_GEMM) {
        *path = PATH_GEMM;
    } else {
        *path = gemv_auto ? PATH_GEMV : PATH_GEMM;
    }
    return CIDER_OK;
}

cider_status run_product(const int8_t *xq, const float *s_tok, const void *wq, const float *s_w,
                         int64_t M, int64_t N, int64_t K, int bits, int group_size,
                         cider::OutKind kind, void *out, void *stream)
{
    cider_status st = check_shape(M, N, K, bits, group_size);
    if (st != CIDER_OK)
        return st;
    if (M == 0 || N == 0)
        return CIDER_OK;
    const bool scaled = kind != cider::OUT_I32;
    if (!xq || !wq || !out || (scaled && (!s_tok || !s_w)))
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(out) || (scaled && !aligned16(s_w)))
        return CIDER_ERR_MISALIGNED;
    int path = PATH_GEMM;
    st = pick_path(M, N, K, bits, group_size, kind, &path);
    if (st != CIDER_OK)
        return st;
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    cider::ProductArgs a{};
    a.xq = xq;
    a.s_tok = s_tok;
    a.wq = wq;
    a.s_w = s_w;
    a.M = M;
    a.N = N;
    a.K = K;
    a.bits = bits;
    a.group_size = group_size;
    a.out_kind = kind;
    a.out = out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(path == PATH_GEMV ? cider::launch_gemv(a, s) : cider::launch_gemm(a, s));
}

bool dtype_ok(int d) { return d == CIDER_DTYPE_F16 || d == CIDER_DTYPE_BF16; }

cider::OutKind out_kind_of(int y_dtype)
{
    return y_dtype == CIDER_DTYPE_BF16 ? cider::OUT_BF16 : cider::OUT_F16;
}

// The whole layer.  static_ws: ignore ws / ws_bytes and use the current
// device's scratch array instead (after every argument and device check).
cider_status run_linear(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        const float *smooth, const void *wq, const float *s_w, int64_t N, int bits,
                        int group_size, int y_dtype, void *ws, size_t ws_bytes, void *y,
                        void *stream, bool static_ws = false)
{
    cider_status st = check_shape(M, N, K, bits, group_size);
    if (st != CIDER_OK)
        return st;
    if (ldx < K || !dtype_ok(x_dtype) || !dtype_ok(y_dtype))
        return CIDER_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return CIDER_OK;
    if (!x || !wq || !s_w || !y)
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(wq) || !aligned16(s_w) || !aligned16(y) || ldx % 8 != 0 ||
        (smooth && !aligned16(smooth)))
        return CIDER_ERR_MISALIGNED;
    int path = PATH_GEMM;
    st = pick_path(M, N, K, bits, group_size, out_kind_of(y_dtype), &path);
    if (st != CIDER_OK)
        return st;
    // Calls in the matrix-vector kernel's earlier automatic range (up to 8
    // int8-weight or 4 int4-weight tokens) may come without a workspace:
    // those keep that kernel, which needs none.
    if (path == PATH_GEMM && !static_ws && (!ws || ws_bytes < cider_linear_workspace_bytes(M, K)) &&
        g_path.load(std::memory_order_relaxed) == PATH_AUTO && M <= (bits == 4 ? 4 : 8) &&
        M * K <= kGemvMaxBytes)
        path = PATH_GEMV;
    // fp16 tokens without smoothing on the matrix-vector path: quantized inside
    // the matrix-vector kernel, whose buffer descriptor spans the tokens with
    // 32-bit byte offsets; a row stride that puts the last token 2 GiB or more
    // past the first goes through the quantize kernel (64-bit row addresses)
    const bool fused = path == PATH_GEMV && x_dtype == CIDER_DTYPE_F16 && !smooth &&
                       ((M - 1) * ldx + K) * 2 < (int64_t(1) << 31);
    if (!fused) {
        if (static_ws) {
            if (cider_linear_workspace_bytes(M, K) > CIDER_NOALLOC_SCRATCH_BYTES)
                return CIDER_ERR_SCRATCH_LIMIT;
        } else {
            if (!ws || ws_bytes < cider_linear_workspace_bytes(M, K))
                return CIDER_ERR_WORKSPACE;
            if (!aligned16(ws))
                return CIDER_ERR_MISALIGNED;
        }
    }
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    if (static_ws && !fused) {
        ws = scratch_address();
        if (!ws)
            return CIDER_ERR_HIP;
        ws_bytes = CIDER_NOALLOC_SCRATCH_BYTES;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused)
        return from_hip(cider::launch_gemv_fused(static_cast<const uint16_t *>(x), M, K, ldx, wq, s_w,
                                                 N, bits, group_size, y, nullptr, nullptr,
                                                 out_kind_of(y_dtype), s));
    int8_t *xq = static_cast<int8_t *>(ws);
    float *s_tok = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + round256((size_t)(M * K)));
    // Split K when the plan asks for it and the workspace has room for the
    // partial sums and tile counters (the quantize launch clears the counters).
    cider::SplitPlan plan{1, 0, 0};
    void *part = nullptr;
    uint32_t *cnt = nullptr;
    if (path == PATH_GEMM) {
        plan = cider::plan_split(M, N, K, bits, group_size);
        if (plan.splits > 1 && ws_bytes >= cider_linear_workspace_bytes(M, K) + split_bytes(plan)) {
            part = static_cast<uint8_t *>(ws) + cider_linear_workspace_bytes(M, K);
            cnt = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(part) + split_part_bytes(plan));
        } else {
            plan.splits = 1;
        }
    }
    hipError_t e = cider::launch_quantize_rows(static_cast<const uint16_t *>(x), x_dtype, M, K, ldx,
                                               smooth, 8, xq, s_tok, s, cnt,
                                               cnt ? (int)plan.tiles : 0);
    if (e != hipSuccess)
        return CIDER_ERR_HIP;
    cider::ProductArgs a{};
    a.xq = xq;
    a.s_tok = s_tok;
    a.wq = wq;
    a.s_w = s_w;
    a.M = M;
    a.N = N;
    a.K = K;
    a.bits = bits;
    a.group_size = group_size;
    a.out_kind = out_kind_of(y_dtype);
    a.out = y;
    if (plan.splits > 1)
        return from_hip(cider::launch_gemm_split(a, plan, part, cnt, s));
    return from_hip(path == PATH_GEMV ? cider::launch_gemv(a, s) : cider::launch_gemm(a, s));
}

cider_status run_quantize_weight(const void *w_f16, int w_dtype, int64_t N, int64_t K, int bits,
                                 int group_size, double clip_percentile, void *wq, float *s_w,
                                 void *stream)
{
    if (N < 0 || K <= 0 || (bits != 8 && bits != 4) || !dtype_ok(w_dtype))
        return CIDER_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return CIDER_ERR_INVALID_ARG;
    if (!(clip_percentile > 0.0 && clip_percentile <= 100.0))  // NaN fails too
        return CIDER_ERR_INVALID_ARG;
    if (K % 64 != 0 || K > kMaxK || (group_size && K % group_size != 0))
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    if (N == 0)
        return CIDER_OK;
    if (!w_f16 || !wq || !s_w)
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(w_f16) || !aligned16(wq) || (reinterpret_cast<uintptr_t>(s_w) & 3u))
        return CIDER_ERR_MISALIGNED;
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    const int64_t len = group_size ? group_size : K;
    const int64_t rows = N * (K / len);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t *w = static_cast<const uint16_t *>(w_f16);
    if (clip_percentile == 100.0)
        return from_hip(cider::launch_quantize_rows(w, w_dtype, rows, len, len, nullptr, bits, wq,
                                                    s_w, s));
    // fractional rank h = (len - 1) * (p / 100) in fp64, as numpy.percentile
    const double h = (double)(len - 1) * (clip_percentile / 100.0);
    const double j = std::floor(h);
    const int64_t r0 = (int64_t)j;
    const int64_t r1 = r0 + 1 < len ? r0 + 1 : len - 1;
    return from_hip(cider::launch_clip_quantize_rows(w, w_dtype, rows, len, r0, r1, h - j, bits, wq,
                                                     s_w, s));
}

}  // namespace

extern "C" {

int cider_is_available(void) { return device_usable(); }

const char *cider_status_str(int status)
{
    switch (status) {
    case CIDER_OK: return "ok";
    case CIDER_ERR_INVALID_ARG: return "invalid argument";
    case CIDER_ERR_UNSUPPORTED_SHAPE: return "shape outside the supported envelope";
    case CIDER_ERR_MISALIGNED: return "pointer or stride not 16-byte aligned";
    case CIDER_ERR_NO_DEVICE: return "no usable gfx950 device";
    case CIDER_ERR_HIP: return "HIP runtime error at launch";
    case CIDER_ERR_WORKSPACE: return "workspace missing or too small";
    case CIDER_ERR_SCRATCH_LIMIT: return "call needs more than the static scratch array holds";
    default: return "unknown status";
    }
}

cider_status cider_quantize_weight(const void *w_f16, int64_t N, int64_t K, int bits,
                                   int group_size, void *wq, float *s_w, void *stream)
{
    return run_quantize_weight(w_f16, CIDER_DTYPE_F16, N, K, bits, group_size, 100.0, wq, s_w,
                               stream);
}

cider_status cider_quantize_weight_clipped(const void *w_f16, int64_t N, int64_t K, int bits,
                                           int group_size, double clip_percentile, void *wq,
                                           float *s_w, void *stream)
{
    return run_quantize_weight(w_f16, CIDER_DTYPE_F16, N, K, bits, group_size, clip_percentile, wq,
                               s_w, stream);
}

cider_status cider_quantize_weight_ex(const void *w, int w_dtype, int64_t N, int64_t K, int bits,
                                      int group_size, double clip_percentile, void *wq, float *s_w,
                                      void *stream)
{
    return run_quantize_weight(w, w_dtype, N, K, bits, group_size, clip_percentile, wq, s_w,
                               stream);
}

cider_status cider_smooth_fold_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                      const float *smooth, void *w_out, void *stream)
{
    if (N < 0 || K <= 0 || !dtype_ok(w_dtype))
        return CIDER_ERR_INVALID_ARG;
    if (K % 8 != 0)
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    if (N == 0)
        return CIDER_OK;
    if (!w || !smooth || !w_out)
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(smooth) || !aligned16(w_out))
        return CIDER_ERR_MISALIGNED;
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    return from_hip(cider::launch_smooth_fold(static_cast<const uint16_t *>(w), w_dtype, N, K, smooth,
                                              static_cast<uint16_t *>(w_out),
                                              static_cast<hipStream_t>(stream)));
}

cider_status cider_quantize_act_ex(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const float *smooth, int8_t *xq, float *s_tok, void *stream)
{
    if (M < 0 || K <= 0 || ldx < K || !dtype_ok(x_dtype))
        return CIDER_ERR_INVALID_ARG;
    if (K % 64 != 0 || K > kMaxK)
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    if (M == 0)
        return CIDER_OK;
    if (!x || !xq || !s_tok)
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || ldx % 8 != 0 ||
        (reinterpret_cast<uintptr_t>(s_tok) & 3u) || (smooth && !aligned16(smooth)))
        return CIDER_ERR_MISALIGNED;
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    return from_hip(cider::launch_quantize_rows(static_cast<const uint16_t *>(x), x_dtype, M, K, ldx,
                                                smooth, 8, xq, s_tok,
                                                static_cast<hipStream_t>(stream)));
}

cider_status cider_quantize_act(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                int8_t *xq, float *s_tok, void *stream)
{
    return cider_quantize_act_ex(x_f16, CIDER_DTYPE_F16, M, K, ldx, nullptr, xq, s_tok, stream);
}

cider_status cider_w8a8_gemm(const int8_t *xq, const float *s_tok, const int8_t *wq,
                             const float *s_w, int64_t M, int64_t N, int64_t K, int group_size,
                             void *y_f16, void *stream)
{
    return run_product(xq, s_tok, wq, s_w, M, N, K, 8, group_size, cider::OUT_F16, y_f16, stream);
}

cider_status cider_w4a8_gemm(const int8_t *xq, const float *s_tok, const uint8_t *wq4,
                             const float *s_w, int64_t M, int64_t N, int64_t K, int group_size,
                             void *y_f16, void *stream)
{
    return run_product(xq, s_tok, wq4, s_w, M, N, K, 4, group_size, cider::OUT_F16, y_f16, stream);
}

cider_status cider_gemm_ex(const int8_t *xq, const float *s_tok, const void *wq, const float *s_w,
                           int64_t M, int64_t N, int64_t K, int bits, int group_size, int y_dtype,
                           void *y, void *stream)
{
    if (!dtype_ok(y_dtype))
        return CIDER_ERR_INVALID_ARG;
    return run_product(xq, s_tok, wq, s_w, M, N, K, bits, group_size, out_kind_of(y_dtype), y,
                       stream);
}

cider_status cider_w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N,
                                 int64_t K, int group_size, int32_t *acc, void *stream)
{
    return run_product(xq, nullptr, wq, nullptr, M, N, K, 8, group_size, cider::OUT_I32, acc,
                       stream);
}

cider_status cider_w4a8_gemm_i32(const int8_t *xq, const uint8_t *wq4, int64_t M, int64_t N,
                                 int64_t K, int group_size, int32_t *acc, void *stream)
{
    return run_product(xq, nullptr, wq4, nullptr, M, N, K, 4, group_size, cider::OUT_I32, acc,
                       stream);
}

size_t cider_linear_workspace_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0)
        return 0;
    return round256((size_t)(M * K)) + round256((size_t)M * sizeof(float));
}

size_t cider_linear_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int bits, int group_size)
{
    const size_t base = cider_linear_workspace_bytes(M, K);
    int path = PATH_GEMM;
    if (check_shape(M, N, K, bits, group_size) != CIDER_OK || M <= 0 || N <= 0 ||
        pick_path(M, N, K, bits, group_size, cider::OUT_F16, &path) != CIDER_OK || path != PATH_GEMM)
        return base;
    const cider::SplitPlan p = cider::plan_split(M, N, K, bits, group_size);
    return p.splits < 2 ? base : base + split_bytes(p);
}

cider_status cider_w8a8_linear(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                               const int8_t *wq, const float *s_w, int64_t N, int group_size,
                               void *workspace, size_t workspace_bytes, void *y_f16, void *stream)
{
    return run_linear(x_f16, CIDER_DTYPE_F16, M, K, ldx, nullptr, wq, s_w, N, 8, group_size,
                      CIDER_DTYPE_F16, workspace, workspace_bytes, y_f16, stream);
}

cider_status cider_w4a8_linear(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                               const uint8_t *wq4, const float *s_w, int64_t N, int group_size,
                               void *workspace, size_t workspace_bytes, void *y_f16, void *stream)
{
    return run_linear(x_f16, CIDER_DTYPE_F16, M, K, ldx, nullptr, wq4, s_w, N, 4, group_size,
                      CIDER_DTYPE_F16, workspace, workspace_bytes, y_f16, stream);
}

cider_status cider_linear_ex(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const float *smooth, const void *wq, const float *s_w, int64_t N,
                             int bits, int group_size, int y_dtype, void *workspace,
                             size_t workspace_bytes, void *y, void *stream)
{
    return run_linear(x, x_dtype, M, K, ldx, smooth, wq, s_w, N, bits, group_size, y_dtype,
                      workspace, workspace_bytes, y, stream);
}

cider_status cider_linear_ex_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                     const float *smooth, const void *wq, const float *s_w,
                                     int64_t N, int bits, int group_size, int y_dtype, void *y,
                                     void *stream)
{
    return run_linear(x, x_dtype, M, K, ldx, smooth, wq, s_w, N, bits, group_size, y_dtype,
                      nullptr, 0, y, stream, true);
}

cider_status cider_decode_linear(const void *x_f16, int64_t K, const void *wq, const float *s_w,
                                 int64_t N, int bits, int group_size, int y_dtype, void *y,
                                 void *stream)
{
    if (N < 0 || K <= 0 || (bits != 8 && bits != 4) || !dtype_ok(y_dtype))
        return CIDER_ERR_INVALID_ARG;
    if (group_size != 0 && group_size != 64 && group_size != 128)
        return CIDER_ERR_INVALID_ARG;
    if (K % 64 != 0 || K > kDecodeMaxK ||
        (group_size && K % group_size != 0))
        return CIDER_ERR_UNSUPPORTED_SHAPE;
    if (N == 0)
        return CIDER_OK;
    if (!x_f16 || !wq || !s_w || !y)
        return CIDER_ERR_INVALID_ARG;
    if (!aligned16(x_f16) || !aligned16(wq) || (reinterpret_cast<uintptr_t>(s_w) & 3u) ||
        (reinterpret_cast<uintptr_t>(y) & 1u))
        return CIDER_ERR_MISALIGNED;
    if (!device_usable())
        return CIDER_ERR_NO_DEVICE;
    return from_hip(cider::launch_decode(static_cast<const uint16_t *>(x_f16), K, wq, s_w, N, bits,
                                         group_size, out_kind_of(y_dtype), y,
                                         static_cast<hipStream_t>(stream)));
}

int cider_set_path(int path)
{
    if (path < 0 || path > 2)
        return -1;
    return g_path.exchange(path);
}

}  // extern "C"
