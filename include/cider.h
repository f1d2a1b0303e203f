/*
 * cider.h -- C ABI of the fused quantized linear layer for AMD Instinct MI355X
 * (gfx950): online per-token INT8 activation quantization, INT8 x INT8 -> INT32
 * matrix product on the matrix cores, and a fused dequantization to fp16.
 *
 * The operation (Cider README, ossradar.top repo page):
 *   - "Modes" table: W8A8 = INT8 symmetric weights x INT8 per-token
 *     activations; W4A8 = INT4 weights packed in uint8 x INT8 per-token
 *     activations.
 *   - "W8A8 Quantization Granularity" table: weights per output channel, or
 *     per group of 64 / 128 input elements.  The pages give W4A8 per column
 *     only; this library also offers W4A8 per group of 64 / 128, the same
 *     groups with int4 codes (one int4 scale per group).
 *   - "Quantization" table: symmetric INT8 activations per token, INT32
 *     accumulation, output C_fp16 = C_int32 * s_act * s_weight per element;
 *     W4A8 weights symmetric INT4 with zero-point 8.
 *   - "Metal Kernel Pipeline": prefill quantizes FP16 activations to INT8 plus
 *     per-token scales, then runs INT8 x INT8 -> INT32 -> FP16 with the scales
 *     applied in the same kernel; a one-token call goes to a matrix-vector
 *     kernel.
 *   - "Low-Level API" / "Layer-level API": quantize_weight_int8(W) -> (w_int8,
 *     scale), pack_weight_int4(W) -> (packed, scale), perchannel_linear(x, w,
 *     scale), w4a8_linear(x, packed, scale); group_size = 0 means per channel.
 *
 * Definitions used by every call (the pages give the granularity, not the
 * arithmetic; these are the readings this library implements):
 *   scale      s = absmax / 127 (int8) or absmax / 7 (int4), fp32, correctly
 *              rounded division; s = 0 for an all-zero row / group.
 *   code       q = clamp(rint(x / s), -127, 127) (int8) or clamp(.., -8, 7)
 *              (int4), x / s a correctly rounded fp32 division, rint rounding
 *              half to even; q = 0 when s = 0.
 *   int4 pack  nibble u = q + 8; byte j of a row holds k = 2j in bits 0..3
 *              and k = 2j + 1 in bits 4..7.
 *   product    acc[m, n] = sum_k xq[m, k] * q_w[n, k] in int32 (exact; needs
 *              K * 127^2 < 2^31, i.e. K <= 133144).  Per group g of gs
 *              elements: acc_g[m, n] = the same sum over k in [g*gs, (g+1)*gs).
 *   output     per channel: y = fp16(acc * s_tok[m] * s_w[n]);
 *              per group:   y = fp16(s_tok[m] * sum_g s_w[n, g] * acc_g),
 *              evaluated in fp32 and rounded to nearest even.
 *
 * Layouts (all row-major, element strides in elements):
 *   x      fp16 [M, K], row stride ldx >= K        (activations, tokens x in)
 *   xq     int8 [M, K], row stride K               (quantized activations)
 *   s_tok  fp32 [M]                                 (per-token scales)
 *   w      fp16 [N, K]                              (nn.Linear weight, out x in)
 *   wq     int8 [N, K]  (bits 8)  or  uint8 [N, K/2] packed (bits 4)
 *   s_w    fp32 [N] (group_size 0) or [N, K/group_size] (group_size 64/128)
 *   y      fp16 [M, N]
 *
 * Ownership and threading: every pointer is device memory owned by the
 * caller; the library allocates, frees and synchronizes nothing.  Work is
 * enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream).  The library keeps no state between calls except the
 * cached device check and the path override below; calls are thread-safe.
 *
 * Errors: every call checks its arguments on the host before touching the
 * HIP runtime and returns a cider_status.  Nothing is launched when the
 * status is not CIDER_OK, except CIDER_ERR_HIP (a launch failed).  Inputs
 * are assumed finite; NaN or Inf inputs give unspecified codes.
 *
 * Envelope: M >= 0 (M = 0 is a no-op), N >= 0 with N % 64 == 0, K > 0 with
 * K % 64 == 0 and K <= 133144, (M + 256) * K < 2^31 and (N + 256) * K < 2^31
 * for the products, group_size in {0, 64, 128} for W8A8 and W4A8;
 * device pointers 16-byte aligned; ldx % 8 == 0.
 */
#ifndef CIDER_H
#define CIDER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CIDER_OK = 0,
    CIDER_ERR_INVALID_ARG = 1,       /* null pointer, negative size, ldx < K, bits or group_size not allowed */
    CIDER_ERR_UNSUPPORTED_SHAPE = 2, /* outside the envelope: K % 64, N % 64, K % group_size, K too large */
    CIDER_ERR_MISALIGNED = 3,        /* a pointer not 16-byte aligned, or ldx % 8 != 0 */
    CIDER_ERR_NO_DEVICE = 4,         /* no usable gfx950 device (or CIDER_FORCE_UNAVAILABLE=1) */
    CIDER_ERR_HIP = 5,               /* the HIP runtime reported an error at launch */
    CIDER_ERR_WORKSPACE = 6,         /* workspace missing or smaller than cider_linear_workspace_bytes */
    CIDER_ERR_SCRATCH_LIMIT = 7      /* cider_linear_ex_noalloc: the call needs more than
                                        CIDER_NOALLOC_SCRATCH_BYTES of workspace */
} cider_status;

/* Element type of 16-bit activations, weights and outputs (Cider README
   feature list: automatic dtype handling, float16 / bfloat16).  Values of
   either type are widened exactly to fp32; outputs are rounded once from the
   fp32 result to nearest even. */
typedef enum {
    CIDER_DTYPE_F16 = 0,
    CIDER_DTYPE_BF16 = 1
} cider_dtype;

/* 1 if the current HIP device is a gfx950 GPU that the library can use, else 0.
   Never crashes: returns 0 when the runtime finds no device.  The environment
   variable CIDER_FORCE_UNAVAILABLE=1 makes it return 0 (a test hook for the
   degrade-gracefully behaviour of Cider README "Conditional Compilation"). */
int cider_is_available(void);

/* Static English text for a status code (never NULL). */
const char *cider_status_str(int status);

/* Weight quantization (Cider README "Low-Level API": quantize_weight_int8,
   pack_weight_int4; "Quantization" table).
   w: fp16 [N, K].  bits 8: wq int8 [N, K]; bits 4: wq uint8 [N, K/2] packed.
   group_size 0: s_w fp32 [N]; 64 or 128: s_w fp32 [N, K/gs] (for bits 4 each
   group's scale is its absmax / 7 and its codes are packed like a row's). */
cider_status cider_quantize_weight(const void *w_f16, int64_t N, int64_t K, int bits,
                                   int group_size, void *wq, float *s_w, void *stream);

/* Weight quantization with percentile clipping (Cider README, "LLM
   Quantization: Precision vs. Speed" note: a percentile method besides plain
   min-max, clip_percentile=99.9).  As cider_quantize_weight, except that each
   row's (group's) range -- the absmax in s = range / 127 or / 7 -- is the
   clip_percentile-th percentile of its |w|: linear interpolation between the
   order statistics around the fractional rank (n - 1) * p / 100, numpy's
   default method, evaluated in fp64 and rounded to fp32.  Values beyond the
   range saturate at the end codes (+-127; int4: 7 and -8).
   0 < clip_percentile <= 100 (else CIDER_ERR_INVALID_ARG); 100 gives exactly
   cider_quantize_weight's result. */
cider_status cider_quantize_weight_clipped(const void *w_f16, int64_t N, int64_t K, int bits,
                                           int group_size, double clip_percentile, void *wq,
                                           float *s_w, void *stream);

/* Weight quantization for either 16-bit type, with optional percentile
   clipping: cider_quantize_weight / cider_quantize_weight_clipped for a w of
   type w_dtype (bf16 magnitudes order like fp16 ones, so clipping finds the
   same order statistics).  clip_percentile = 100 is plain absmax. */
cider_status cider_quantize_weight_ex(const void *w, int w_dtype, int64_t N, int64_t K, int bits,
                                      int group_size, double clip_percentile, void *wq, float *s_w,
                                      void *stream);

/* SmoothQuant's weight fold (Cider README: SmoothQuant named among the
   preprocessing methods for quantization-friendly models).  With smoothing
   factors s [K] (fp32, positive, 16-byte aligned) the activations are
   divided by s inside cider_quantize_act_ex / cider_linear_ex and the weights
   absorb it offline: w_out[n, k] = w[n, k] * s[k], the exact product rounded
   once to nearest even in w's own type.  w, w_out [N, K] of type w_dtype,
   16-byte aligned; K % 8 == 0; w_out may equal w. */
cider_status cider_smooth_fold_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                      const float *smooth, void *w_out, void *stream);

/* Per-token activation quantization of fp16 or bf16 activations, with an
   optional SmoothQuant smoothing vector smooth [K] (fp32, 16-byte aligned,
   NULL for none): x'[m, k] = fp32(x[m, k] / smooth[k]) (correctly rounded)
   before the absmax, and the codes are those of x'.  Otherwise as
   cider_quantize_act. */
cider_status cider_quantize_act_ex(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const float *smooth, int8_t *xq, float *s_tok, void *stream);

/* Per-token activation quantization (Cider README "Metal Kernel Pipeline",
   step quantize_per_token; "Quantization" table, Activations row).
   x: fp16 [M, K] with row stride ldx.  xq: int8 [M, K]; s_tok: fp32 [M]. */
cider_status cider_quantize_act(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                int8_t *xq, float *s_tok, void *stream);

/* W8A8 product with fused dequantization (Cider README "Metal Kernel
   Pipeline", step matmul_fused_dequant; "TensorOps matmul2d"; "W8A8
   Quantization Granularity").  group_size 0: per-channel s_w [N];
   64 / 128: per-group s_w [N, K/gs].  y: fp16 [M, N].
   Under the automatic path setting the matrix-vector kernel takes
   M * K <= 65536 with M <= 3 per channel or M <= 2 per group where the
   few-token matrix-core kernel applies (K a multiple of 128 int8 / 256 int4
   values), else M <= 8 (M <= 4 for int4 weights); everything else runs the
   matrix-core kernels. */
cider_status cider_w8a8_gemm(const int8_t *xq, const float *s_tok, const int8_t *wq,
                             const float *s_w, int64_t M, int64_t N, int64_t K,
                             int group_size, void *y_f16, void *stream);

/* W4A8 product (Cider README "Modes": Unpack -> TensorOps; "Metal Kernel
   Pipeline": INT4 -> INT8 unpacking before the INT8 product).
   wq4: uint8 [N, K/2] packed nibbles.  group_size 0: s_w fp32 [N];
   64 / 128: per-group s_w fp32 [N, K/gs] (the per-group output formula). */
cider_status cider_w4a8_gemm(const int8_t *xq, const float *s_tok, const uint8_t *wq4,
                             const float *s_w, int64_t M, int64_t N, int64_t K,
                             int group_size, void *y_f16, void *stream);

/* Either product (bits 8: wq int8 [N, K]; bits 4: packed uint8 [N, K/2]) with
   the output rounded to y_dtype (fp16 or bf16): y [M, N]. */
cider_status cider_gemm_ex(const int8_t *xq, const float *s_tok, const void *wq, const float *s_w,
                           int64_t M, int64_t N, int64_t K, int bits, int group_size, int y_dtype,
                           void *y, void *stream);

/* Test hooks: the same kernels with the dequant epilogue replaced by a raw
   store of the int32 accumulators ("Quantization" table, Accumulation INT32):
   acc int32 [M, N] (group_size 0) or [M, N, K/gs] (one sum per group). */
cider_status cider_w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N,
                                 int64_t K, int group_size, int32_t *acc, void *stream);
cider_status cider_w4a8_gemm_i32(const int8_t *xq, const uint8_t *wq4, int64_t M, int64_t N,
                                 int64_t K, int group_size, int32_t *acc, void *stream);

/* Bytes of device workspace cider_w8a8_linear / cider_w4a8_linear need for M
   tokens of K features (the int8 activations and their scales). */
size_t cider_linear_workspace_bytes(int64_t M, int64_t K);

/* Bytes of workspace that also let a linear call of this shape split K over
   several workgroups per output tile (2 to 8 splits on the matrix-core path,
   where that is faster: per group up to 256 tokens; per channel never): the
   int8 activations and scales as above, then the partial sums of the split
   product (4 bytes per output of each 64 x 32, 64 or 128 tile and split) and
   one counter per tile. Equal to cider_linear_workspace_bytes(M, K) when the
   shape is not split, shapes the matrix-vector kernel serves under the
   current path setting included. The split count follows the current
   device's compute-unit count. A linear call given at least this many bytes
   splits; given fewer (but at least cider_linear_workspace_bytes(M, K)) it
   runs unsplit. The fp32 partial sums of the splits are added in split order
   (deterministic; a different rounding order from the unsplit group-by-group
   sum, within the same tolerance of the exact result). */
size_t cider_linear_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int bits,
                                       int group_size);

/* The whole layer on fp16 activations, mirroring perchannel_linear(x, w, s)
   and w4a8_linear(x, packed, s) of Cider README "Low-Level API":
   quantize_act into `workspace`, then the product.  On the matrix-vector path
   the quantization is fused into the matrix-vector kernel and the workspace
   is not touched (it may be null).  Under the automatic path setting that
   path takes M * K <= 65536 with M <= 3 per channel or M <= 2 per group
   where the few-token matrix-core kernel applies (K a multiple of 128 for
   int8 weights, 256 for int4), else M <= 8 (M <= 4 for int4 weights); calls
   within M <= 8 (int4: 4) and M * K <= 65536 given no workspace, or less
   than cider_linear_workspace_bytes(M, K), also take it.  x: fp16 [M, K]
   row stride ldx; y: fp16 [M, N]. */
cider_status cider_w8a8_linear(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                               const int8_t *wq, const float *s_w, int64_t N, int group_size,
                               void *workspace, size_t workspace_bytes, void *y_f16,
                               void *stream);
cider_status cider_w4a8_linear(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                               const uint8_t *wq4, const float *s_w, int64_t N, int group_size,
                               void *workspace, size_t workspace_bytes, void *y_f16,
                               void *stream);

/* The whole layer for any input / output type, with optional smoothing:
   cider_quantize_act_ex into `workspace`, then cider_gemm_ex.  fp16 tokens
   without smoothing on the matrix-vector path (see cider_w8a8_linear) are
   quantized inside the matrix-vector kernel and need no workspace; every
   other call needs cider_linear_workspace_bytes(M, K) bytes of it, or cider_linear_workspace_bytes_ex(...) bytes to split K.
   Calls that share a workspace must be ordered (one stream). */
cider_status cider_linear_ex(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const float *smooth, const void *wq, const float *s_w, int64_t N,
                             int bits, int group_size, int y_dtype, void *workspace,
                             size_t workspace_bytes, void *y, void *stream);

/* Size of the static device array that serves as cider_linear_ex_noalloc's
   workspace on each GPU (64 MiB). */
#define CIDER_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): the same
   layer as cider_linear_ex, with the workspace taken from a file-scope device
   array of CIDER_NOALLOC_SCRATCH_BYTES per GPU that the library holds until
   the process ends.  No allocation of any kind happens in the call; the
   first call on a device looks up that device's array address once.  The
   call splits K exactly when cider_linear_ex given
   cider_linear_workspace_bytes_ex(...) bytes would, as long as those bytes fit
   in the array, so its results equal that call's bit for bit; shapes whose
   split workspace does not fit run unsplit (equal to cider_linear_ex given
   cider_linear_workspace_bytes(M, K) bytes).  Calls whose
   cider_linear_workspace_bytes(M, K) exceeds the array (M * K above about
   64 Mi) return CIDER_ERR_SCRATCH_LIMIT before any launch; fused one-token
   calls use no workspace.  Every call on one GPU shares that GPU's array and
   leaves its contents behind (the quantize launch clears the split counters
   each call), so calls must be ordered on one stream: calls that overlap on
   one GPU (concurrent streams, several host threads) race on the array and
   give undefined results.  Arguments and other statuses as cider_linear_ex. */
cider_status cider_linear_ex_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                     const float *smooth, const void *wq, const float *s_w,
                                     int64_t N, int bits, int group_size, int y_dtype, void *y,
                                     void *stream);

/* The pages' decode kernel (Cider README, "Metal Kernel Pipeline", Decode
   (M = 1): a direct matrix-vector product with on-the-fly weight
   dequantization and no activation quantization):
     y[n] = sum_g s_w[n, g] * sum_{k in g} x[k] * q[n, k]
   (per channel: one group of K), accumulated in fp32 and rounded once to
   y_dtype.  x fp16 [K]; wq / s_w as for the products (bits 8 or 4, group_size
   0 / 64 / 128); y [N].  K % 64 == 0 and K <= 32768; any N >= 0.  Unlike the W8A8 one-token path, the result is not
   that of the quantized-activation formula: it is the dequantized-weight
   product, the other reading of the pages' decode step. */
cider_status cider_decode_linear(const void *x_f16, int64_t K, const void *wq, const float *s_w,
                                 int64_t N, int bits, int group_size, int y_dtype, void *y,
                                 void *stream);

/* Test hook: force the product path for subsequent calls in this process.
   0 = automatic (M * K <= 65536 and M <= 8, or M <= 4 for int4 weights ->
   matrix-vector, else matrix cores),
   1 = always the matrix-vector kernel (calls with M > 8 or M * K > 65536 then
   return CIDER_ERR_UNSUPPORTED_SHAPE), 2 = always the matrix-core kernel.
   Returns the previous setting, or -1 for an invalid value. */
int cider_set_path(int path);

#ifdef __cplusplus
}
#endif

#endif /* CIDER_H */
