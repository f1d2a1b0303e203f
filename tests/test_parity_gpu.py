"""GPU parity: the HIP kernels against the oracle, element by element.

Bit-exact: quantized activations and their scales, quantized weights and
their scales, int32 accumulators (through the _i32 hooks).  fp16 outputs:
|y - y_ref| <= 1e-3 + 2^-10 |y_ref|.  Shapes span several tiles of both
kernel paths with ragged tails in M and N (N stays a multiple of 64, the
documented envelope), and the degenerate cases: zero rows, exact ties, a
single token, the long-row quantize kernel, and identical results from the
matrix-vector and matrix-core paths on the same inputs."""
import numpy as np
import pytest

import synth_inputs as si
import w4a8_quantized_linear_amd as cider
from oracle.oracle import get as get_oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MODES = [(8, 0), (8, 64), (8, 128), (4, 0), (4, 64), (4, 128)]
MODE_IDS = ["w8a8_pc", "w8a8_pg64", "w8a8_pg128", "w4a8_pc", "w4a8_pg64", "w4a8_pg128"]


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert cider.cider_is_available(), "libcider.so reports no usable gfx950 device"
    cider.cider_set_path(cider.PATH_AUTO)
    yield
    cider.cider_set_path(cider.PATH_AUTO)


@pytest.fixture(autouse=True)
def _announce(request):
    gu.announce(request.node.nodeid)
    yield
    cider.cider_set_path(cider.PATH_AUTO)


# ---------------------------------------------------------------- quantize ---

ACT_SHAPES = [(64, 1024, 1024), (37, 2560, 2624), (5, 10240, 10240), (3, 12288, 12288),
              (2, 20480, 20480), (1, 64, 64), (1000, 128, 136), (9, 4096, 4096),
              (7, 6144, 6152), (11, 8192, 8200), (4, 16384, 16384), (600, 10240, 10240)]


@pytest.mark.parametrize("M,K,ldx", ACT_SHAPES)
def test_quantize_act_bitexact(M, K, ldx):
    orc = get_oracle()
    x = si.activations(M, ldx, seed=M + K)
    if M >= 3:
        x[1] = 0                                   # all-zero token
        x[2, :] = np.float16(0.5)                  # ties at scale 1
        x[2, 7] = np.float16(-127.0)
        x[2, 8:16] = np.array([1.5, 2.5, -0.5, -2.5, 126.5, 3.25, -3.75, 0.0], np.float16)
    xd = gu.to_dev(x)
    xq, st = gu.quantize_act_gpu(xd, M, K, ldx)
    rq, rs = orc.quantize_act(x, K=K)
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)


def _near_half_rows(amaxes, K=640):
    """One row per absmax A: A itself and, for every half-integer h + 0.5 below
    127, the fp16 values nearest (h + 0.5) * s and their two neighbours on each
    side (s = fl32(A / 127)), signs alternating; zeros after.  Quotients at or
    within a few ulps of a half-integer, where the rounding of x / s decides
    the code."""
    rows, ties = [], 0
    for A in amaxes:
        a16 = np.float16(A)
        s = np.float32(a16) / np.float32(127.0)
        vals = [a16]
        for h in range(127):
            base = np.array([(h + 0.5) * float(s)], np.float16).view(np.uint16)[0]
            for d in (-2, -1, 0, 1, 2):
                b = int(base) + d
                if 0 <= b <= int(np.array([a16]).view(np.uint16)[0]):
                    vals.append(np.array([b], np.uint16).view(np.float16)[0])
        row = np.zeros(K, np.float16)
        v = np.array(vals[:K], np.float16)
        v[1::2] = -v[1::2]
        row[:len(v)] = v
        q32 = np.abs(row.astype(np.float32) / s)
        ties += int(np.sum(q32 - np.floor(q32) == 0.5))
        rows.append(row)
    return np.stack(rows), ties


NEAR_HALF_AMAX = [1.0, 0.7, 3.0, 100.0, 65504.0, 2.0 ** -10, 2.0 ** -14, 0.3337, 12.34] + list(
    2.0 ** np.random.default_rng(17).uniform(-14.0, 15.9, 119))


def test_quantize_near_half_quotients():
    """Codes where fl32(x / s) sits on or next to a half-integer: the kernel's
    rounding of the quotient must match the oracle's bit for bit (both the
    per-token quantize kernel and, through an identity weight, the fused
    one-token path)."""
    orc = get_oracle()
    x, ties = _near_half_rows(NEAR_HALF_AMAX)
    assert ties > 0, "the rows must contain exact half-integer quotients"
    M, K = x.shape
    xq, st = gu.quantize_act_gpu(gu.to_dev(x), M, K, K)
    rq, rs = orc.quantize_act(x, K=K)
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)
    # fused path: y = 127 q s_tok s_w for an identity weight, one token at a time
    eye = np.eye(K, dtype=np.float16)
    wq, sw = orc.quantize_weight(eye, 8, 0)
    wd, swd = gu.to_dev(wq), gu.to_dev(sw)
    for i in range(M):
        row = x[i:i + 1]
        y = gu.to_host(gu.linear_gpu(gu.to_dev(row), 1, K, K, wd, swd, K, 8, 0))
        ref, rxq, _ = orc.linear(row, wq, sw, 8, 0, K=K)
        assert np.array_equal(rxq, rq[i:i + 1])
        gu.assert_f16_close(y, ref, "near-half row %d" % i)


WEIGHT_CASES = [(512, 1024, 8, 0), (512, 1024, 8, 64), (512, 1024, 8, 128), (512, 1024, 4, 0),
                (10240, 2560, 8, 0), (2560, 10240, 8, 64), (2560, 10240, 8, 128),
                (10240, 2560, 4, 0), (64, 20480, 8, 0), (64, 20480, 4, 0),
                (512, 1024, 4, 64), (512, 1024, 4, 128), (2560, 10240, 4, 64),
                (2560, 10240, 4, 128), (512, 4096, 8, 0), (256, 8192, 4, 0)]


@pytest.mark.parametrize("N,K,bits,gs", WEIGHT_CASES)
def test_quantize_weight_bitexact(N, K, bits, gs):
    orc = get_oracle()
    w = si.weights(N, K)
    w[3, :] = 0
    if gs:
        w[5, :gs] = 0
    wq, sw = gu.quantize_weight_gpu(w, bits, gs)
    rq, rs = orc.quantize_weight(w, bits, gs)
    assert np.array_equal(gu.to_host(sw), rs)
    assert np.array_equal(gu.to_host(wq), rq)


CLIP_CASES = [(512, 1024, 8, 0), (512, 1024, 8, 64), (512, 1024, 8, 128), (512, 1024, 4, 0),
              (512, 1024, 4, 64), (512, 1024, 4, 128), (10240, 2560, 8, 0), (2560, 10240, 8, 64),
              (2560, 10240, 4, 128), (64, 20480, 8, 0), (128, 10240, 4, 0)]


@pytest.mark.parametrize("p", [99.9, 99.0, 50.0, 100.0])
@pytest.mark.parametrize("N,K,bits,gs", CLIP_CASES)
def test_quantize_weight_clipped_bitexact(N, K, bits, gs, p):
    """Percentile clipping: codes and scales bit-exact, with rows / groups of
    zeros, of many ties, of 99.9% zeros (range 0) and a row of equal values."""
    if N * K > 4 * 2 ** 20 and p not in (99.9,):
        pytest.skip("full-size shapes at the default percentile only")
    import torch
    orc = get_oracle()
    w = si.weights(N, K, seed=N + K)
    L = gs if gs else K
    w[3, :] = 0
    w[5, :] = np.round(w[5, :].astype(np.float32) * 100) / 100     # many ties
    w[6, :] = 0
    w[6, 7] = np.float16(0.5)                                       # one nonzero per row
    w[7, :L] = np.float16(-0.03)                                    # one value repeated
    wd = gu.to_dev(w)
    wq = gu.empty((N, K) if bits == 8 else (N, K // 2), torch.int8 if bits == 8 else torch.uint8)
    sw = gu.empty((N,) if gs == 0 else (N, K // gs), torch.float32)
    cider.cider_quantize_weight_clipped(wd, N, K, bits, gs, p, wq, sw)
    rq, rs = orc.quantize_weight_clipped(w, bits, gs, p)
    assert np.array_equal(gu.to_host(sw), rs)
    assert np.array_equal(gu.to_host(wq), rq)
    if p == 100.0:
        pq, ps = orc.quantize_weight(w, bits, gs)
        assert np.array_equal(rq, pq) and np.array_equal(rs, ps)


# ------------------------------------------------- bf16 and smoothing ---

def _smoothing(K, seed):
    rng = np.random.default_rng([seed, 77])
    return rng.uniform(0.05, 20.0, K).astype(np.float32)


@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("M,K,ldx", [(64, 1024, 1024), (37, 2560, 2624), (5, 10240, 10240),
                                     (3, 20480, 20480), (130, 256, 264), (1, 64, 64),
                                     (600, 6144, 6144)])
def test_quantize_act_ex_bitexact(M, K, ldx, dtype, smooth):
    """fp16 / bf16 activations, with and without a smoothing vector:
    codes and scales bit-exact (including a zero token and exact ties)."""
    orc = get_oracle()
    x = si.activations(M, ldx, seed=M + K).astype(np.float32)
    if M >= 3:
        x[1] = 0
        x[2, :16] = [0.5, 1.5, 2.5, -0.5, -2.5, 126.5, 3.25, -3.75, 0.0, -127.0, 1, 2, 3, 4, 5, 6]
    xb = gu.bf16_bits(x) if dtype == 1 else x.astype(np.float16).view(np.uint16)
    sm = _smoothing(K, M) if smooth else None
    import torch
    xq = gu.empty((M, K), torch.int8)
    st = gu.empty((M,), torch.float32)
    smd = gu.to_dev(sm) if smooth else None
    cider.cider_quantize_act_ex(gu.bits_to_dev(xb), dtype, M, K, ldx, smd, xq, st)
    rq, rs = orc.quantize_act_ex(xb, dtype, K=K, smooth=sm)
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)


@pytest.mark.parametrize("p", [100.0, 99.9])
@pytest.mark.parametrize("N,K,bits,gs", [(512, 1024, 8, 0), (512, 1024, 4, 64), (512, 1024, 8, 128),
                                         (2560, 10240, 4, 128), (10240, 2560, 8, 0)])
def test_quantize_weight_bf16_bitexact(N, K, bits, gs, p):
    import torch
    orc = get_oracle()
    wb = gu.bf16_bits(si.weights(N, K, seed=N).astype(np.float32))
    wb[3] = 0
    wq = gu.empty((N, K) if bits == 8 else (N, K // 2), torch.int8 if bits == 8 else torch.uint8)
    sw = gu.empty((N,) if gs == 0 else (N, K // gs), torch.float32)
    cider.cider_quantize_weight_ex(gu.bits_to_dev(wb), 1, N, K, bits, gs, p, wq, sw)
    rq, rs = orc.quantize_weight_ex(wb, 1, bits, gs, p)
    assert np.array_equal(gu.to_host(sw), rs)
    assert np.array_equal(gu.to_host(wq), rq)


# Row magnitudes whose fp32 scale is not a normal number: absmax / 127 below
# 2^-126 (and for 2^-133, the smallest bf16, a scale whose reciprocal
# overflows).  1e-30 stays normal, as a control.
TINY_AMAX = [1e-36, 3e-37, 1e-38, 2.0 ** -133, 1e-30]


def _tiny_rows(amaxes, K, seed):
    """float32 rows of N(0,1) values rescaled to the given absmax, each with
    zeros, +-absmax, +-absmax/2 and +-absmax/4 at fixed positions."""
    rng = np.random.default_rng([seed, 5])
    rows = []
    for a in amaxes:
        r = rng.standard_normal(K).astype(np.float64)
        r = r / np.abs(r).max() * a
        r[:8] = [0.0, a, -a, a / 2, -a / 2, a / 4, 0.0, -a]
        rows.append(r.astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("K", [64, 256, 1024, 2560, 10240, 20480])
def test_quantize_act_tiny_scales_bitexact(K):
    """bf16 tokens whose scale is subnormal in fp32 (and one whose reciprocal
    overflows), mixed with ordinary tokens: codes and scales bit-exact.  K
    spans every team size of the quantize kernel and its long-row kernel."""
    import torch
    orc = get_oracle()
    x = np.concatenate([_tiny_rows(TINY_AMAX, K, K), si.activations(3, K, seed=K).astype(np.float32)])
    xb = gu.bf16_bits(x)
    M = xb.shape[0]
    xq = gu.empty((M, K), torch.int8)
    st = gu.empty((M,), torch.float32)
    cider.cider_quantize_act_ex(gu.bits_to_dev(xb), 1, M, K, K, None, xq, st)
    rq, rs = orc.quantize_act_ex(xb, 1, K=K)
    assert np.any((rs > 0) & (rs < 2.0 ** -126)), "the rows must give subnormal scales"
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)


@pytest.mark.parametrize("K", [256, 1024, 10240, 20480])
def test_quantize_act_huge_smoothing_bitexact(K):
    """fp16 tokens divided by smoothing factors of 1e38 .. 3e38: the smoothed
    values, and so the scales, fall below the normal fp32 range (tokens 2-3
    scaled by 1/64 give scales whose reciprocal overflows); codes and scales
    bit-exact against the oracle."""
    import torch
    orc = get_oracle()
    x = si.activations(6, K, seed=K)
    x[1, :8] = np.array([0, 1, -1, 0.5, -0.5, 0.25, 0, 3], np.float16)
    x[2:4] = (x[2:4].astype(np.float32) / 64).astype(np.float16)
    xb = x.view(np.uint16)
    sm = (np.random.default_rng([K, 9]).uniform(1.0, 3.0, K) * 1e38).astype(np.float32)
    M = x.shape[0]
    xq = gu.empty((M, K), torch.int8)
    st = gu.empty((M,), torch.float32)
    cider.cider_quantize_act_ex(gu.bits_to_dev(xb), 0, M, K, K, gu.to_dev(sm), xq, st)
    rq, rs = orc.quantize_act_ex(xb, 0, K=K, smooth=sm)
    assert np.all(rs < 2.0 ** -126), "the smoothed rows must give subnormal scales"
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)


@pytest.mark.parametrize("p", [100.0, 99.9])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
def test_quantize_weight_bf16_tiny_scales_bitexact(bits, gs, p):
    """bf16 weight rows (and groups) whose scale, absmax / 127 or / 7, is
    subnormal in fp32: codes and scales bit-exact."""
    import torch
    orc = get_oracle()
    N, K = 64, 1024
    w = si.weights(N, K, seed=3).astype(np.float32)
    w[:len(TINY_AMAX)] = _tiny_rows(TINY_AMAX, K, 11)
    w[8:8 + len(TINY_AMAX)] = _tiny_rows(TINY_AMAX, K, 12) * 7.0 / 127.0
    if gs:
        w[20, :gs] = _tiny_rows([1e-37], gs, 13)[0]          # one tiny group in a normal row
    wb = gu.bf16_bits(w)
    wq = gu.empty((N, K) if bits == 8 else (N, K // 2), torch.int8 if bits == 8 else torch.uint8)
    sw = gu.empty((N,) if gs == 0 else (N, K // gs), torch.float32)
    cider.cider_quantize_weight_ex(gu.bits_to_dev(wb), 1, N, K, bits, gs, p, wq, sw)
    rq, rs = orc.quantize_weight_ex(wb, 1, bits, gs, p)
    assert np.any((rs > 0) & (rs < 2.0 ** -126))
    assert np.array_equal(gu.to_host(sw), rs)
    assert np.array_equal(gu.to_host(wq), rq)


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("N,K", [(512, 1024), (2560, 10240), (64, 8)])
def test_smooth_fold_bitexact(N, K, dtype):
    """w * s_k rounded once to the weight type, bit-exact; also in place."""
    orc = get_oracle()
    w = si.weights(N, K, seed=K).astype(np.float32)
    wb = gu.bf16_bits(w) if dtype == 1 else w.astype(np.float16).view(np.uint16)
    sm = _smoothing(K, N)
    sm[:4] = [1.0, 2.0 ** -20, 3.0e4, 0.5]      # identity, tiny (subnormal products), large
    ref = orc.smooth_fold_weight(wb, dtype, sm)
    wd = gu.bits_to_dev(wb)
    out = gu.bits_to_dev(np.zeros_like(wb))
    cider.cider_smooth_fold_weight(wd, dtype, N, K, gu.to_dev(sm), out)
    assert np.array_equal(gu.bits_to_host(out), ref)
    cider.cider_smooth_fold_weight(wd, dtype, N, K, gu.to_dev(sm), wd)
    assert np.array_equal(gu.bits_to_host(wd), ref)


@pytest.mark.parametrize("path", [cider.PATH_GEMM, cider.PATH_AUTO])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 512, 1024), (64, 512, 1024), (300, 320, 1024),
                                   (1100, 704, 1024), (200, 192, 1344)])
def test_product_bf16_output(M, N, K, bits, gs, path):
    """bf16 outputs of every product kernel within one bf16 ulp of the
    oracle (which rounds the exact dequant once)."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    cider.cider_set_path(path)
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M * 5 + N)
    y = gu.empty((M, N), torch.int16)
    cider.cider_gemm_ex(gu.to_dev(xq), gu.to_dev(st), gu.to_dev(wq), gu.to_dev(sw), M, N, K, bits,
                        gs, 1, y)
    ref = orc.dequant_ex(orc.gemm_acc(xq, wq, bits, gs), st, sw, 1)
    gu.assert_out_close(gu.bits_to_host(y), ref, 1, "bf16 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("x_dtype,y_dtype,smooth", [(1, 1, False), (0, 0, True), (1, 1, True),
                                                    (1, 0, False), (0, 1, False)])
@pytest.mark.parametrize("M,N,K,ldx", [(1, 512, 1024, 1024), (1, 2560, 10240, 10240),
                                       (64, 512, 1024, 1088), (130, 640, 2560, 2560)])
def test_linear_ex_whole_path(M, N, K, ldx, x_dtype, y_dtype, smooth, bits, gs):
    """The whole layer for bf16 / fp16 inputs and outputs, with SmoothQuant
    smoothing (activations divided inside the quantizer, weights folded by
    the library's fold kernel), against the oracle's whole path."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    orc = get_oracle()
    x = si.activations(M, ldx, seed=K).astype(np.float32)
    xb = gu.bf16_bits(x) if x_dtype == 1 else x.astype(np.float16).view(np.uint16)
    w = si.weights(N, K, seed=K)
    sm = _smoothing(K, 3) if smooth else None
    wbits = w.view(np.uint16)
    if smooth:
        wbits = orc.smooth_fold_weight(wbits, 0, sm)
        wd = gu.bits_to_dev(w.view(np.uint16))
        cider.cider_smooth_fold_weight(wd, 0, N, K, gu.to_dev(sm), wd)
        assert np.array_equal(gu.bits_to_host(wd), wbits)
    wq, sw = orc.quantize_weight(wbits.view(np.float16), bits, gs)
    ws_bytes = cider.cider_linear_workspace_bytes(M, K)
    ws = gu.empty((max(ws_bytes, 16),), torch.uint8)
    y = gu.empty((M, N), torch.int16)
    cider.cider_linear_ex(gu.bits_to_dev(xb), x_dtype, M, K, ldx, gu.to_dev(sm) if smooth else None,
                          gu.to_dev(wq), gu.to_dev(sw), N, bits, gs, y_dtype, ws, ws_bytes, y)
    ref, _, _ = orc.linear_ex(xb, x_dtype, wq, sw, bits, gs, K=K, smooth=sm, y_dtype=y_dtype)
    gu.assert_out_close(gu.bits_to_host(y), ref, y_dtype, "linear_ex M=%d" % M)


# ------------------------------------------------------- decode variant ---

DECODE_SHAPES = [(512, 1024), (10240, 2560), (2560, 10240), (100, 640), (64, 16384), (3, 64)]


@pytest.mark.parametrize("y_dtype", [0, 1])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("N,K", DECODE_SHAPES + [(64, 32768)])
def test_decode_linear(N, K, bits, gs, y_dtype):
    """The decode variant (dequantized weights, fp16 activation as is) against
    the oracle's fp64 evaluation.  The kernel sums in fp32, so the bound adds
    2^-16 of the sum of |terms| to the usual output tolerance (the fp32
    summation error of at most ~100 sequential additions is below 2^-17 of it)."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    orc = get_oracle()
    x = si.activations(1, K, seed=N + K)[0]
    w = si.weights(N, K, seed=N)
    wq, sw = orc.quantize_weight(w, bits, gs)
    y = gu.empty((N,), torch.int16)
    cider.cider_decode_linear(gu.to_dev(x), K, gu.to_dev(wq), gu.to_dev(sw), N, bits, gs, y_dtype, y)
    ref = orc.decode_linear(x, 0, wq, sw, bits, gs, y_dtype)
    codes = wq.astype(np.float64) if bits == 8 else gu.unpack_int4(wq).astype(np.float64)
    L = K if gs == 0 else gs
    swf = np.repeat(np.asarray(sw, np.float64).reshape(N, -1), L, axis=1)
    S = (np.abs(codes) * swf) @ np.abs(x.astype(np.float64))
    got = gu.bits_to_f64(gu.bits_to_host(y), y_dtype)
    r = gu.bits_to_f64(ref, y_dtype)
    bound = 1e-3 + (2.0 ** -10 if y_dtype == 0 else 2.0 ** -7) * np.abs(r) + 2.0 ** -16 * S
    err = np.abs(got - r)
    assert np.all(np.isfinite(got)) and np.all(err <= bound), (
        "%d of %d outside, worst ratio %.3g" % (int((err > bound).sum()), N, float((err / bound).max())))


# ----------------------------------------------------------------- product ---

# (100 / 200 / 256 tokens at K = 1024 / 2048: per group, the few-token
# kernel's 32-token tiles repeated over M, or with int8 weights past 192
# tokens the persistent per-group tiles)
PRODUCT_SHAPES = [(64, 512, 1024), (300, 320, 1024), (700, 576, 512), (513, 1024, 2560),
                  (1, 512, 1024), (17, 64, 128), (1100, 704, 1024), (2100, 320, 1024),
                  (40, 320, 576), (200, 192, 1344), (100, 320, 1024), (200, 320, 1024),
                  (256, 640, 2048)]


def _inputs(M, N, K, bits, gs, seed):
    x = si.activations(M, K, seed=seed)
    w = si.weights(N, K, seed=seed)
    orc = get_oracle()
    wq, sw = orc.quantize_weight(w, bits, gs)
    xq, st = orc.quantize_act(x)
    return x, w, xq, st, wq, sw


@pytest.mark.parametrize("path", [cider.PATH_GEMM, cider.PATH_AUTO])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", PRODUCT_SHAPES)
def test_product_i32_bitexact(M, N, K, bits, gs, path):
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    cider.cider_set_path(path)
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M * 7 + N)
    acc = gu.gemm_i32_gpu(gu.to_dev(xq), gu.to_dev(wq), M, N, K, bits, gs)
    ref = orc.gemm_acc(xq, wq, bits, gs)
    assert np.array_equal(gu.to_host(acc), ref)


@pytest.mark.parametrize("path", [cider.PATH_GEMM, cider.PATH_AUTO])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", PRODUCT_SHAPES)
def test_product_f16_tolerance(M, N, K, bits, gs, path):
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    cider.cider_set_path(path)
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M * 7 + N)
    y = gu.gemm_gpu(gu.to_dev(xq), gu.to_dev(st), gu.to_dev(wq), gu.to_dev(sw), M, N, K, bits, gs)
    ref = orc.dequant(orc.gemm_acc(xq, wq, bits, gs), st, sw)
    gu.assert_f16_close(gu.to_host(y), ref, "M=%d N=%d K=%d bits=%d gs=%d" % (M, N, K, bits, gs))


@pytest.mark.parametrize("out", ["i32", "f16", "bf16"])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", [(16, 8256, 512), (32, 10240, 2560), (24, 8192, 256),
                                   (9, 192, 1024), (32, 2560, 10240), (31, 64, 768), (5, 128, 256)])
def test_few_token_kernel(M, N, K, bits, gs, out):
    """The few-token product (up to 32 tokens, ragged in M): 64-channel tiles
    from N = 8192, 16-channel tiles below, one or two 16-token blocks, one to
    twenty K units per K-split wavefront, int8 / int4 weights, per channel and
    per group; int32 sums bit-exact (the per-group int32 hook takes another
    kernel), fp16 / bf16 outputs within tolerance of the oracle."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    cider.cider_set_path(cider.PATH_GEMM)
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M * 11 + N)
    acc = orc.gemm_acc(xq, wq, bits, gs)
    what = "M=%d N=%d K=%d bits=%d gs=%d %s" % (M, N, K, bits, gs, out)
    if out == "i32":
        got = gu.gemm_i32_gpu(gu.to_dev(xq), gu.to_dev(wq), M, N, K, bits, gs)
        assert np.array_equal(gu.to_host(got), acc), what
        return
    dt = 0 if out == "f16" else 1
    y = gu.empty((M, N), torch.int16)
    cider.cider_gemm_ex(gu.to_dev(xq), gu.to_dev(st), gu.to_dev(wq), gu.to_dev(sw), M, N, K, bits,
                        gs, dt, y)
    gu.assert_out_close(gu.bits_to_host(y), orc.dequant_ex(acc, st, sw, dt), dt, what)


@pytest.mark.parametrize("out", ["i32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,N,K", [(2100, 10304, 1024), (1100, 640, 256), (1030, 576, 1344),
                                   (1100, 320, 128), (4100, 704, 2560), (1100, 5056, 1024),
                                   (1100, 10176, 512), (2040, 10176, 256), (4000, 6080, 256),
                                   (160, 2112, 1024), (224, 2176, 1024), (450, 2240, 1024),
                                   (700, 2240, 1024), (900, 2304, 1024)])
def test_many_token_tiles(M, N, K, bits, out):
    """Per-channel persistent tiles.  With K a multiple of 128 and at least
    256, one workgroup per compute unit walks output tiles.  On a 256-unit
    device: 2100 x 10304 takes two rounds of 256 x 256 tiles (369, so some
    workgroups take two; ragged in M and N); 1100 x 10176 one round of
    256 x 256 (200); 2040 x 10176 one round of 320 x 256 (256), where
    256 x 256 would need two; 1100 x 5056 one round of 160 x 256 (160) but
    not of 160 x 128 (288); 1100 x 640 and 4100 x 704 one round of 160 x 128
    (36 and 165, ragged N); 4000 x 6080 two whole rounds of 192 x 256 with
    int8 weights (512, ragged in M and N), where 256 x 256 and 320 x 256
    would leave the second round partly empty; deep-K tiles of the other
    kernel from 129 to 512 tokens: 160 x 2112 64 x 64 tiles (99 workgroups,
    ragged M), 224 x 2176 128 x 128 tiles (34, ragged in M and N) and, int8
    only, 450 x 2240 128 x 192 tiles (54, ragged in M and N), 700 x 2240
    128 x 256 tiles (54, ragged M; int4 with 128-value K tiles) and
    900 x 2304 160 x 256 tiles (60, ragged in M and N).  K = 1344 (not a multiple of 128) and K = 128
    (one K tile) take the other kernel.  int32 sums bit-exact and outputs
    within tolerance on sampled rows against the oracle, every output
    against the exact product."""
    import torch
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, 0, seed=M + N + K)
    d = [gu.to_dev(a) for a in (xq, st, wq, sw)]
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 511, M // 2, M - 2, M - 1],
                                     np.random.default_rng(M).integers(0, M, 8)]))
    rows = rows[rows < M]
    ref_acc = orc.gemm_acc(xq[rows], wq, bits, 0)
    if out == "i32":
        acc = gu.to_host(gu.gemm_i32_gpu(d[0], d[2], M, N, K, bits, 0))
        assert np.array_equal(acc[rows], ref_acc)
        full = xq.astype(np.int64) @ (wq if bits == 8 else gu.unpack_int4(wq)).astype(np.int64).T
        assert np.array_equal(acc, full)
        return
    y_dtype = 0 if out == "f16" else 1
    y = gu.empty((M, N), torch.int16)
    cider.cider_gemm_ex(d[0], d[1], d[2], d[3], M, N, K, bits, 0, y_dtype, y)
    got = gu.bits_to_host(y)
    gu.assert_out_close(got[rows], orc.dequant_ex(ref_acc, st[rows], sw, y_dtype), y_dtype,
                        "%s M=%d N=%d K=%d bits=%d" % (out, M, N, K, bits))
    if out == "f16":
        gu.assert_every_output(y.view(torch.float16), xq, st, wq if bits == 8 else gu.unpack_int4(wq), sw, 0,
                               "M=%d N=%d K=%d bits=%d" % (M, N, K, bits))


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("bits,gs", [(8, 128), (4, 128), (8, 64), (4, 64)])
@pytest.mark.parametrize("M,N,K", [(4100, 2624, 1024), (3100, 640, 2048), (3100, 640, 1344)])
def test_many_token_tiles_per_group(M, N, K, bits, gs, out):
    """Per-group products with many tokens.  4100 x 2624: too many tiles for
    one round even at 256 channels, so int8 groups of 128 take the 320 x 128
    persistent kernel (297 output tiles, ragged in M and N, so some
    workgroups take two), int8 groups of 64 the other kernel, and int4
    weights the 192 x 256 persistent tiles with two token blocks per wave
    (238 tiles, ragged in M and N); 3100 x 640: one
    round of 64 x 128 persistent tiles (250 of them, ragged in M); K = 1344
    (not a multiple of 128) takes the other kernel.  Sampled rows against the
    oracle, every output against the exact product."""
    if K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M + N + K + gs)
    d = [gu.to_dev(a) for a in (xq, st, wq, sw)]
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, M // 2, M - 2, M - 1],
                                     np.random.default_rng(M + gs).integers(0, M, 8)]))
    y_dtype = 0 if out == "f16" else 1
    y = gu.empty((M, N), torch.int16)
    cider.cider_gemm_ex(d[0], d[1], d[2], d[3], M, N, K, bits, gs, y_dtype, y)
    got = gu.bits_to_host(y)
    ref = orc.dequant_ex(orc.gemm_acc(xq[rows], wq, bits, gs), st[rows], sw, y_dtype)
    gu.assert_out_close(got[rows], ref, y_dtype, "%s M=%d N=%d K=%d bits=%d gs=%d" % (out, M, N, K, bits, gs))
    if out == "f16":
        gu.assert_every_output(y.view(torch.float16), xq, st, wq if bits == 8 else gu.unpack_int4(wq), sw, gs,
                               "M=%d N=%d K=%d bits=%d gs=%d" % (M, N, K, bits, gs))


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("bits,gs", MODES[1:3] + MODES[4:6], ids=MODE_IDS[1:3] + MODE_IDS[4:6])
@pytest.mark.parametrize("M,N,K", [(1030, 1984, 1024), (1300, 2496, 1024), (1100, 3776, 1024),
                                   (2100, 3008, 1024)])
def test_mid_token_tiles_per_group(M, N, K, bits, gs, out):
    """Per-group persistent tiles with more than one channel block per wave
    row, ragged in M and N.  On a 256-unit device: 1030 x 1984 takes one
    round of 128 x 96 tiles (176; 64 x 128 would need 279); 1300 x 2496 of
    128 x 128 (220; 128 x 96 would need 280); 1100 x 3776 of 192 x 128 (180;
    128 x 128 would need 270); 2100 x 3008 of 256 x 128 (204; 192 x 128
    would need 272).  (The 64-channel tiles are reached by the product tests'
    shapes.)  Sampled rows against the oracle, every output against the
    exact product."""
    import torch
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M + N + K + gs + bits)
    d = [gu.to_dev(a) for a in (xq, st, wq, sw)]
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, M // 2, M - 2, M - 1],
                                     np.random.default_rng(M + gs).integers(0, M, 8)]))
    y_dtype = 0 if out == "f16" else 1
    y = gu.empty((M, N), torch.int16)
    cider.cider_gemm_ex(d[0], d[1], d[2], d[3], M, N, K, bits, gs, y_dtype, y)
    got = gu.bits_to_host(y)
    ref = orc.dequant_ex(orc.gemm_acc(xq[rows], wq, bits, gs), st[rows], sw, y_dtype)
    gu.assert_out_close(got[rows], ref, y_dtype, "%s M=%d N=%d K=%d bits=%d gs=%d" % (out, M, N, K, bits, gs))
    if out == "f16":
        gu.assert_every_output(y.view(torch.float16), xq, st, wq if bits == 8 else gu.unpack_int4(wq), sw, gs,
                               "M=%d N=%d K=%d bits=%d gs=%d" % (M, N, K, bits, gs))


@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 512, 1024), (3, 320, 2560), (8, 576, 4096), (2, 128, 10240)])
def test_gemv_path_matches_gemm_path(M, N, K, bits, gs):
    """The matrix-vector kernel (forced for M <= 8) and the matrix-core kernel
    give identical int32 sums and fp16 outputs within tolerance."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    orc = get_oracle()
    _, _, xq, st, wq, sw = _inputs(M, N, K, bits, gs, seed=M + 3)
    d = [gu.to_dev(a) for a in (xq, st, wq, sw)]
    ref_acc = orc.gemm_acc(xq, wq, bits, gs)
    ref_y = orc.dequant(ref_acc, st, sw)
    for path in (cider.PATH_GEMV, cider.PATH_GEMM):
        cider.cider_set_path(path)
        acc = gu.gemm_i32_gpu(d[0], d[2], M, N, K, bits, gs)
        assert np.array_equal(gu.to_host(acc), ref_acc), "path %d" % path
        y = gu.gemm_gpu(d[0], d[1], d[2], d[3], M, N, K, bits, gs)
        gu.assert_f16_close(gu.to_host(y), ref_y, "path %d" % path)


# ------------------------------------------------------------------ linear ---

@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K,ldx", [(1, 512, 1024, 1024), (1, 10240, 2560, 2560),
                                       (1, 2560, 10240, 10240), (64, 512, 1024, 1088),
                                       (130, 640, 2560, 2560)])
def test_linear_whole_path(M, N, K, ldx, bits, gs):
    """fp16 activations in, fp16 out: quantization fused into the one-token
    kernel at M = 1, through the workspace otherwise."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    orc = get_oracle()
    x = si.activations(M, ldx, seed=K)
    w = si.weights(N, K, seed=K)
    wq, sw = orc.quantize_weight(w, bits, gs)
    y = gu.linear_gpu(gu.to_dev(x), M, K, ldx, gu.to_dev(wq), gu.to_dev(sw), N, bits, gs)
    ref, _, _ = orc.linear(x, wq, sw, bits, gs, K=K)
    gu.assert_f16_close(gu.to_host(y), ref, "linear M=%d" % M)


@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", [(2, 10240, 2560), (3, 2560, 10240), (4, 10240, 2560),
                                   (6, 2560, 10240), (8, 10240, 2560)])
def test_linear_few_tokens_auto(M, N, K, bits, gs):
    """The automatic path at 2..8 tokens: given the workspace, the few-token
    matrix-core kernel from 4 tokens per channel / 3 per group (the
    matrix-vector kernel below); given none, the matrix-vector kernel with the
    tokens quantized inside it wherever M * K <= 65536 (int4: M <= 4), and a
    workspace error past that.  Both against the oracle's whole layer."""
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    cider.cider_set_path(cider.PATH_AUTO)
    orc = get_oracle()
    x = si.activations(M, K, seed=M + K)
    w = si.weights(N, K, seed=N)
    wq, sw = orc.quantize_weight(w, bits, gs)
    ref, _, _ = orc.linear(x, wq, sw, bits, gs, K=K)
    xd, wqd, swd = gu.to_dev(x), gu.to_dev(wq), gu.to_dev(sw)
    y = gu.linear_gpu(xd, M, K, K, wqd, swd, N, bits, gs)
    gu.assert_f16_close(gu.to_host(y), ref, "linear M=%d with workspace" % M)
    f = cider.cider_w8a8_linear if bits == 8 else cider.cider_w4a8_linear
    y0 = gu.empty((M, N), torch.float16)
    st = f(xd, M, K, K, wqd, swd, N, gs, None, 0, y0, check=False)
    if M * K <= 65536 and M <= (4 if bits == 4 else 8):
        assert st == cider.CIDER_OK
        gu.assert_f16_close(gu.to_host(y0), ref, "linear M=%d without workspace" % M)
    else:
        assert st == cider.CIDER_ERR_WORKSPACE


def test_deterministic_repeats():
    """Integer results are identical across repeated launches (no races in
    the LDS staging)."""
    M, N, K = 1024, 1024, 2560
    _, _, xq, st, wq, sw = _inputs(M, N, K, 8, 0, seed=5)
    d = [gu.to_dev(a) for a in (xq, wq)]
    a1 = gu.to_host(gu.gemm_i32_gpu(d[0], d[1], M, N, K, 8, 0))
    a2 = gu.to_host(gu.gemm_i32_gpu(d[0], d[1], M, N, K, 8, 0))
    assert np.array_equal(a1, a2)


def test_quality_report_small_workload():
    """Quality of the quantized layer against the fp16 product on the small
    per-channel workload (M=64, N=512, K=1024, seed 0): reported; the value
    is a property of the quantization scheme on these inputs."""
    x = si.activations(64, 1024)
    w = si.weights(512, 1024)
    wq, sw = gu.quantize_weight_gpu(w, 8, 0)
    y = gu.to_host(gu.linear_gpu(gu.to_dev(x), 64, 1024, 1024, wq, sw, 512, 8, 0))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    cos = gu.cosine(y, ref)
    gu.announce("cosine vs fp16 product, W8A8 per-channel 64x512x1024: %.5f" % cos)
    assert cos > 0.998
