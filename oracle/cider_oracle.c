/*
 * cider_oracle.c -- plain CPU reference for the fused quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * library: it is a second, independent statement of what the layer computes.
 *
 * What is computed, and where the pages say so:
 *   Cider README (ossradar.top repo page), "Quantization" table:
 *     - activations: symmetric INT8, one scale per token (row of X);
 *     - W8A8 weights: symmetric INT8, per output channel or per group of
 *       64/128 consecutive input elements;
 *     - W4A8 weights: symmetric INT4 with zero-point 8, stored packed in uint8;
 *     - accumulation in INT32;
 *     - output dequant: C_fp16 = C_int32 * s_act * s_weight, per element.
 *   Same README, "W8A8 Quantization Granularity" table (per-channel = one scale
 *   per output channel; per-group = one scale per 64 or 128 elements) and the
 *   "LLM Quantization: Precision vs. Speed" note (scales by plain min-max).
 *   Same README, "Metal Kernel Pipeline": FP16 activations -> INT8 + per-token
 *   scales, then INT8 x INT8 -> INT32 -> FP16.
 *   Same README: automatic dtype handling (float16 / bfloat16) among the
 *   features; SmoothQuant named as the preprocessing that makes activations
 *   quantization-friendly (activations divided per input channel by a
 *   smoothing factor, the weights multiplied by it).
 *
 * Readings taken where the pages are silent:
 *   - scale s = absmax / 127 (int8) or absmax / 7 (int4), computed in fp32;
 *   - code q = clamp(round_half_even(fp32(x / s)), lo, hi), the quotient a
 *     correctly rounded fp32 division; int8 range [-127, 127], int4 [-8, 7];
 *   - an all-zero row or group gets s = 0 and q = 0;
 *   - int4 nibble u = q + 8 (zero-point 8); byte j of a packed row holds
 *     k = 2j in its low nibble and k = 2j + 1 in its high nibble;
 *   - per-group scales are stored [N, K / group_size], row-major;
 *   - percentile clipping (weights only): the range replacing the absmax is
 *     the numpy-default linear-interpolation percentile of |w| over the row
 *     or group, computed in fp64 and rounded to fp32;
 *   - bf16 activations / weights are widened exactly like fp16 ones;
 *   - smoothing: x' = fp32(x / smooth[k]) before the absmax; the weight fold
 *     is w' = w * smooth[k] exactly, rounded once to the weight's type;
 *   - dequant is evaluated in fp64 and rounded once to fp16 or bf16 (round to
 *     nearest even, overflow to infinity).  Per-group:
 *     y = s_tok * sum_g s_w[n,g]*acc_g.
 *
 * Quantization decisions are taken in fp32 because the scales are fp32
 * values; everything after the integer accumulation is fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (oracle.py, compile_oracle).
 * Rows are split across OpenMP threads; the arithmetic per row is the plain
 * loop written below, in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_OVERFLOW = 2 };

/* Element types of activations, weights and outputs. */
enum { DT_F16 = 0, DT_BF16 = 1 };

/* K > 0; bits 8 or 4; group_size 0 (per channel) or a divisor of K; int4
   packs two codes per byte, so K is even. */
static int shape_ok(int64_t K, int bits, int group_size)
{
    if (K <= 0 || (bits != 8 && bits != 4))
        return 0;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0))
        return 0;
    if (bits == 4 && K % 2 != 0)
        return 0;
    return 1;
}

/* ---------------------------------------------------------------- fp16 --- */

/* Exact widening of an IEEE binary16 bit pattern. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)man, -24);              /* zero / subnormal: man * 2^-24 */
    else if (e == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), e - 25);  /* (1 + man/1024) * 2^(e - 15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even; overflow -> inf. */
uint16_t oracle_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    /* 65520 is the midpoint between 65504 (largest finite) and 65536 (which
       would be the next binade); ties go to the even neighbour, 65536 = inf. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    /* Quantum (distance between neighbouring halves) at a: 2^-24 below the
       smallest normal 2^-14, else 2^(e-11) where a = f * 2^e, f in [0.5, 1). */
    int e = 0;
    frexp(a, &e);
    int q = (a < ldexp(1.0, -14)) ? -24 : e - 11;
    double m = nearbyint(ldexp(a, -q));           /* count of quanta, ties to even */
    if (q == -24)                                  /* subnormal (m == 1024 is 2^-14) */
        return (uint16_t)(sign | (uint16_t)m);
    if (m == 2048.0) {                             /* rounded up into the next binade */
        m = 1024.0;
        q += 1;
    }
    /* value = m * 2^q with m in [1024, 2048): biased exponent = q + 25 */
    return (uint16_t)(sign | ((q + 25) << 10) | ((int)m - 1024));
}

float oracle_half_to_float(uint16_t h) { return (float)oracle_half_to_double(h); }

/* --------------------------------------------------------------- bf16 --- */

/* Exact widening of a bfloat16 bit pattern: bfloat16 is the upper half of an
   IEEE binary32, so the pattern shifted into the high 16 bits is the value. */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value, ties to even; overflow -> inf. */
uint16_t oracle_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7fc0);
    /* Quantum at a: 2^-133 below the smallest normal 2^-126, else 2^(e-8)
       where a = f * 2^e, f in [0.5, 1) (8 significant bits). */
    int e = 0;
    frexp(a, &e);
    int q = (a < ldexp(1.0, -126)) ? -133 : e - 8;
    double m = nearbyint(ldexp(a, -q));           /* count of quanta, ties to even */
    if (q == -133)                                 /* subnormal (m == 128 is 2^-126) */
        return (uint16_t)(sign | (uint16_t)m);
    if (m == 256.0) {                              /* rounded up into the next binade */
        m = 128.0;
        q += 1;
    }
    /* value = m * 2^q with m in [128, 256): biased exponent = q + 134 */
    if (q + 134 >= 255)
        return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | ((q + 134) << 7) | ((int)m - 128));
}

static float widen(uint16_t h, int dtype)
{
    return dtype == DT_BF16 ? (float)oracle_bf16_to_double(h) : oracle_half_to_float(h);
}

static uint16_t narrow(double v, int dtype)
{
    return dtype == DT_BF16 ? oracle_double_to_bf16(v) : oracle_double_to_half(v);
}

static int dtype_ok(int dtype) { return dtype == DT_F16 || dtype == DT_BF16; }

/* ------------------------------------------------------- quantization --- */

/* n consecutive fp16 / bf16 values as fp32 (exact).  With a smoothing vector
   (SmoothQuant's per-input-channel factors, one per k), each value is first
   divided by its channel's factor: an fp32 quotient, before any absmax. */
static void widen_run(const uint16_t *x, int dtype, int64_t n, const float *smooth, float *v)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = widen(x[i], dtype);
        v[i] = smooth ? f / smooth[i] : f;
    }
}

static float absmax_of(const float *v, int64_t n)
{
    float absmax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > absmax)
            absmax = a;
    }
    return absmax;
}

/* Symmetric quantization of n fp32 values over the range [-range, range]:
   s = range / qmax, codes clamped to [lo, hi].
   Writes the integer codes to q[0..n) and returns the fp32 scale. */
static float quantize_range(const float *v, int64_t n, float range, float qmax, int lo,
                            int hi, int *q)
{
    float s = range / qmax;                        /* fp32, correctly rounded */
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = v[i] / s;  /* fp32 quotient */
        float r = nearbyintf(t);                   /* round half to even */
        int c = (int)r;
        if (c < lo) c = lo;
        if (c > hi) c = hi;
        q[i] = c;
    }
    return s;
}

static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

/* The p-th percentile (0 < p <= 100) of |v| over n values, by linear
   interpolation between the two order statistics around the fractional rank
   h = (n - 1) * (p / 100) -- the default method of numpy.percentile, whose
   fp64 steps are followed here: a = v[floor(h)], b = the next value (the last
   one past the end), d = b - a, g = h - floor(h); the result is a + d*g for
   g < 0.5 and b - d*(1 - g) otherwise.  buf holds n doubles. */
static double percentile_abs(const float *v, int64_t n, double p, double *buf)
{
    for (int64_t i = 0; i < n; ++i)
        buf[i] = fabs((double)v[i]);
    qsort(buf, (size_t)n, sizeof(double), cmp_double);
    double h = (double)(n - 1) * (p / 100.0);
    double j = floor(h);
    double g = h - j;
    int64_t i0 = (int64_t)j;
    int64_t i1 = i0 + 1 < n ? i0 + 1 : n - 1;
    double a = buf[i0], b = buf[i1];
    double d = b - a;
    return g >= 0.5 ? b - d * (1.0 - g) : a + d * g;
}

/* The same over n fp16 values (exposed for the tests). */
double oracle_percentile_abs(const uint16_t *x, int64_t n, double p, double *buf)
{
    float *v = (float *)malloc((size_t)n * sizeof(float));
    widen_run(x, DT_F16, n, NULL, v);
    double r = percentile_abs(v, n, p, buf);
    free(v);
    return r;
}

/* Per-token activation quantization: X [M, K] (fp16 or bf16) with row stride
   ldx, optionally divided by a smoothing vector smooth [K] first.
   xq int8 [M, K] (row stride K), s_tok fp32 [M]. */
int oracle_quantize_act_ex(const uint16_t *x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           const float *smooth, int8_t *xq, float *s_tok)
{
    if (!x || !xq || !s_tok || M < 0 || K <= 0 || ldx < K || !dtype_ok(dtype))
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float *v = (float *)malloc((size_t)K * sizeof(float));
        int *q = (int *)malloc((size_t)K * sizeof(int));
        widen_run(x + m * ldx, dtype, K, smooth, v);
        s_tok[m] = quantize_range(v, K, absmax_of(v, K), 127.0f, -127, 127, q);
        for (int64_t k = 0; k < K; ++k)
            xq[m * K + k] = (int8_t)q[k];
        free(q);
        free(v);
    }
    return ORACLE_OK;
}

int oracle_quantize_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                        float *s_tok)
{
    return oracle_quantize_act_ex(x, DT_F16, M, K, ldx, NULL, xq, s_tok);
}

/* Weight quantization, W [N, K] (fp16 or bf16, row stride K).
   bits = 8: wq int8 [N, K];   bits = 4: wq uint8 [N, K/2] packed nibbles.
   group_size = 0: one scale per output channel, s_w fp32 [N];
   group_size = g: one scale per (n, k-group of g), s_w fp32 [N, K/g].
   clip_percentile < 100 replaces each run's absmax by that percentile of its
   |w| (Cider README, "LLM Quantization: Precision vs. Speed" note: besides
   plain min-max, a percentile method, clip_percentile=99.9), so the largest
   values saturate at the end codes. */
int oracle_quantize_weight_ex(const uint16_t *w, int dtype, int64_t N, int64_t K, int bits,
                              int group_size, double clip_percentile, uint8_t *wq, float *s_w)
{
    if (!w || !wq || !s_w || N < 0 || !shape_ok(K, bits, group_size) || !dtype_ok(dtype))
        return ORACLE_BAD_ARG;
    if (!(clip_percentile > 0.0 && clip_percentile <= 100.0))
        return ORACLE_BAD_ARG;
    int64_t gs = group_size ? group_size : K;
    int64_t G = K / gs;
    float qmax = bits == 8 ? 127.0f : 7.0f;
    int lo = bits == 8 ? -127 : -8, hi = bits == 8 ? 127 : 7;
    int clip = clip_percentile < 100.0;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int *qbuf = (int *)malloc((size_t)K * sizeof(int));
        float *v = (float *)malloc((size_t)gs * sizeof(float));
        double *buf = clip ? (double *)malloc((size_t)gs * sizeof(double)) : NULL;
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *run = w + n * K + g * gs;
            widen_run(run, dtype, gs, NULL, v);
            /* the range: the run's absmax, or the percentile of its |w| in fp32 */
            float range = clip ? (float)percentile_abs(v, gs, clip_percentile, buf)
                               : absmax_of(v, gs);
            s_w[n * G + g] = quantize_range(v, gs, range, qmax, lo, hi, qbuf + g * gs);
        }
        if (bits == 8) {
            for (int64_t k = 0; k < K; ++k)
                wq[n * K + k] = (uint8_t)(int8_t)qbuf[k];
        } else {
            for (int64_t j = 0; j < K / 2; ++j) {
                int u_even = qbuf[2 * j] + 8;      /* zero-point 8 */
                int u_odd = qbuf[2 * j + 1] + 8;
                wq[n * (K / 2) + j] = (uint8_t)(u_even | (u_odd << 4));
            }
        }
        free(buf);
        free(v);
        free(qbuf);
    }
    return ORACLE_OK;
}

int oracle_quantize_weight(const uint16_t *w, int64_t N, int64_t K, int bits,
                           int group_size, uint8_t *wq, float *s_w)
{
    return oracle_quantize_weight_ex(w, DT_F16, N, K, bits, group_size, 100.0, wq, s_w);
}

int oracle_quantize_weight_clipped(const uint16_t *w, int64_t N, int64_t K, int bits,
                                   int group_size, double clip_percentile, uint8_t *wq,
                                   float *s_w)
{
    return oracle_quantize_weight_ex(w, DT_F16, N, K, bits, group_size, clip_percentile, wq,
                                     s_w);
}

/* SmoothQuant's weight side, folded offline: W' = W diag(smooth), i.e.
   w'[n, k] = w[n, k] * smooth[k], the exact product (fp64 holds it: at most
   11 + 24 significant bits) rounded once, to nearest even, to W's type. */
int oracle_smooth_fold_weight(const uint16_t *w, int dtype, int64_t N, int64_t K,
                              const float *smooth, uint16_t *w_out)
{
    if (!w || !smooth || !w_out || N < 0 || K <= 0 || !dtype_ok(dtype))
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w_out[n * K + k] = narrow((double)widen(w[n * K + k], dtype) * (double)smooth[k], dtype);
    return ORACLE_OK;
}

/* ------------------------------------------------------ accumulation --- */

/* Weight code at (n, k) of a quantized weight, as a signed integer. */
static int weight_code(const uint8_t *wq, int bits, int64_t K, int64_t n, int64_t k)
{
    if (bits == 8)
        return (int8_t)wq[n * K + k];
    uint8_t b = wq[n * (K / 2) + k / 2];
    int u = (k % 2 == 0) ? (b & 0xf) : (b >> 4);
    return u - 8;                                  /* zero-point 8 */
}

/* sum over k in [k0, k1) of xrow[k] * w[n, k], exact in int64. */
static int64_t dot_range(const int8_t *xrow, const uint8_t *wq, int bits, int64_t K,
                         int64_t n, int64_t k0, int64_t k1)
{
    int64_t s = 0;
    for (int64_t k = k0; k < k1; ++k)
        s += (int64_t)xrow[k] * weight_code(wq, bits, K, n, k);
    return s;
}

/* Integer accumulators acc[m, n, g] = sum over k in group g of xq[m,k]*w[n,k].
   acc int32 [M, N, G] with G = 1 (group_size 0) or K / group_size.
   The sums are formed in int64 and must fit int32. */
int oracle_gemm_acc(const int8_t *xq, const uint8_t *wq, int bits, int64_t M,
                    int64_t N, int64_t K, int group_size, int32_t *acc)
{
    if (!xq || !wq || !acc || M < 0 || N < 0 || !shape_ok(K, bits, group_size))
        return ORACLE_BAD_ARG;
    int64_t gs = group_size ? group_size : K;
    int64_t G = K / gs;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t g = 0; g < G; ++g) {
                int64_t s = dot_range(xq + m * K, wq, bits, K, n, g * gs, (g + 1) * gs);
                if (s > INT32_MAX || s < INT32_MIN)
                    overflow = 1;
                acc[(m * N + n) * G + g] = (int32_t)s;
            }
        }
    }
    return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* ------------------------------------------------------------ dequant --- */

/* s_tok * sum_g s_w[g] * acc[g], evaluated in fp64.  With G = 1 this is
   acc * s_tok * s_w, the per-channel form of the 'Output dequant' row. */
static double dequant_value(float s_tok, const float *s_w_row, const int32_t *acc_row, int64_t G)
{
    double t = 0.0;
    for (int64_t g = 0; g < G; ++g)
        t += (double)s_w_row[g] * (double)acc_row[g];
    return (double)s_tok * t;
}

/* y [M, N] (fp16 or bf16, rounded once to nearest even) from acc int32
   [M, N, G], s_tok [M], s_w [N, G]. */
int oracle_dequant_ex(const int32_t *acc, const float *s_tok, const float *s_w, int64_t M,
                      int64_t N, int64_t G, int y_dtype, uint16_t *y)
{
    if (!acc || !s_tok || !s_w || !y || M < 0 || N < 0 || G <= 0 || !dtype_ok(y_dtype))
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = narrow(dequant_value(s_tok[m], s_w + n * G, acc + (m * N + n) * G, G),
                                  y_dtype);
    return ORACLE_OK;
}

int oracle_dequant(const int32_t *acc, const float *s_tok, const float *s_w,
                   int64_t M, int64_t N, int64_t G, uint16_t *y)
{
    return oracle_dequant_ex(acc, s_tok, s_w, M, N, G, DT_F16, y);
}

/* --------------------------------------------------------- whole path --- */

/* X [M, K] (fp16 or bf16, row stride ldx, optionally smoothed) through
   quantize_act, the integer product with an already-quantized weight and the
   dequant, one row at a time.  xq / s_tok receive the quantized activations;
   y [M, N] in y_dtype. */
int oracle_linear_ex(const uint16_t *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const float *smooth, const uint8_t *wq, const float *s_w, int bits,
                     int64_t N, int group_size, int y_dtype, int8_t *xq, float *s_tok,
                     uint16_t *y)
{
    if (!x || !wq || !s_w || !xq || !s_tok || !y || M < 0 || N < 0 || ldx < K ||
        !shape_ok(K, bits, group_size) || !dtype_ok(x_dtype) || !dtype_ok(y_dtype))
        return ORACLE_BAD_ARG;
    int64_t gs = group_size ? group_size : K;
    int64_t G = K / gs;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t m = 0; m < M; ++m) {
        float *v = (float *)malloc((size_t)K * sizeof(float));
        int *q = (int *)malloc((size_t)K * sizeof(int));
        int32_t *accs = (int32_t *)malloc((size_t)G * sizeof(int32_t));
        widen_run(x + m * ldx, x_dtype, K, smooth, v);
        s_tok[m] = quantize_range(v, K, absmax_of(v, K), 127.0f, -127, 127, q);
        for (int64_t k = 0; k < K; ++k)
            xq[m * K + k] = (int8_t)q[k];
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t g = 0; g < G; ++g) {
                int64_t s = dot_range(xq + m * K, wq, bits, K, n, g * gs, (g + 1) * gs);
                if (s > INT32_MAX || s < INT32_MIN)
                    overflow = 1;
                accs[g] = (int32_t)s;
            }
            y[m * N + n] = narrow(dequant_value(s_tok[m], s_w + n * G, accs, G), y_dtype);
        }
        free(accs);
        free(q);
        free(v);
    }
    return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

int oracle_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  const uint8_t *wq, const float *s_w, int bits, int64_t N,
                  int group_size, int8_t *xq, float *s_tok, uint16_t *y)
{
    return oracle_linear_ex(x, DT_F16, M, K, ldx, NULL, wq, s_w, bits, N, group_size, DT_F16, xq,
                            s_tok, y);
}

/* ----------------------------------------------------- decode variant --- */

/* The pages' decode kernel (Cider README, "Metal Kernel Pipeline", Decode
   (M = 1): a direct matrix-vector product that dequantizes the weights on
   the fly and does not quantize the activation):
     y[n] = sum_g s_w[n, g] * (sum over k in group g of x[k] * q[n, k])
   (one group of K for per-channel scales), x fp16 / bf16 [K], evaluated in
   fp64 and rounded once to y_dtype.  Each product x * q is exact in fp64;
   the sums are fp64 in k order. */
int oracle_decode_linear(const uint16_t *x, int x_dtype, int64_t K, const uint8_t *wq,
                         const float *s_w, int bits, int64_t N, int group_size, int y_dtype,
                         uint16_t *y)
{
    if (!x || !wq || !s_w || !y || N < 0 || !shape_ok(K, bits, group_size) ||
        !dtype_ok(x_dtype) || !dtype_ok(y_dtype))
        return ORACLE_BAD_ARG;
    int64_t gs = group_size ? group_size : K;
    int64_t G = K / gs;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double t = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double a = 0.0;
            for (int64_t k = g * gs; k < (g + 1) * gs; ++k)
                a += (double)widen(x[k], x_dtype) * (double)weight_code(wq, bits, K, n, k);
            t += (double)s_w[n * G + g] * a;
        }
        y[n] = narrow(t, y_dtype);
    }
    return ORACLE_OK;
}

/* Threads the OpenMP loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of later calls (n >= 1).  Scheduling only: every
   loop above splits independent rows, so results do not depend on it. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
