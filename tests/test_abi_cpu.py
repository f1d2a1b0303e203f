"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
any HIP call.  No kernel is ever launched here: CIDER_FORCE_UNAVAILABLE=1 is
set for the whole module, so a call with valid arguments stops at the device
check (CIDER_ERR_NO_DEVICE) even on a machine with a GPU.  Pointers passed
are fake integers that are never dereferenced."""
import os
import re

import pytest

import w4a8_quantized_linear_amd as cider

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cider.h")

P = 0x10000          # a 16-byte aligned fake device address
P2 = 0x20000
P3 = 0x30000
P4 = 0x40000
BAD = 0x10008        # 8-byte aligned only


@pytest.fixture(autouse=True)
def _no_device(monkeypatch):
    monkeypatch.setenv("CIDER_FORCE_UNAVAILABLE", "1")
    cider.cider_set_path(cider.PATH_AUTO)
    yield
    cider.cider_set_path(cider.PATH_AUTO)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cider_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = cider.load()
    names = _declared()
    assert len(names) >= 12
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(cider.EXPORTS) == names


def test_unavailable_without_device():
    assert cider.cider_is_available() is False


def test_status_strings():
    for s in range(8):
        assert cider.cider_status_str(s) not in ("", "unknown status")
    assert cider.cider_status_str(99) == "unknown status"


def test_workspace_bytes():
    assert cider.cider_linear_workspace_bytes(0, 64) == 0
    assert cider.cider_linear_workspace_bytes(3, 64) == 256 + 256
    assert cider.cider_linear_workspace_bytes(4096, 2560) == 4096 * 2560 + 16384


def _r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("M,N,K,bits,gs", [(64, 2560, 10240, 8, 64), (48, 2560, 10240, 4, 64),
                                           (128, 64, 10240, 8, 128), (40, 640, 2560, 4, 128),
                                           (100, 320, 1024, 8, 64), (256, 2560, 10240, 8, 64),
                                           (16, 640, 320, 8, 64), (32, 256, 640, 4, 64)])
def test_workspace_bytes_split(M, N, K, bits, gs):
    """The split workspace: activations + scales, then partial sums of whole
    64 x TM tiles (TM = 32 / 64 / 128 by token count) for 2..8 splits (no
    more splits than K units), then one counter per tile."""
    base = cider.cider_linear_workspace_bytes(M, K)
    ex = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
    TM = 32 if M <= 32 else 64 if M <= 64 else 128
    tiles = -(-N // 64) * -(-M // TM)
    fits = [S for S in range(2, 9) if S <= K // gs and
            ex == base + _r256(tiles * S * 64 * TM * 4) + _r256(tiles * 4)]
    assert len(fits) == 1, (ex, base)


def test_workspace_bytes_no_split():
    # per channel never splits; per group from 33 to 256 tokens, and up to 32
    # only where K is not a multiple of the few-token kernel's unit (128
    # values int8, 256 int4)
    for M, N, K, bits, gs in [(16, 2560, 10240, 4, 64), (9, 640, 2560, 4, 128), (32, 2560, 10240, 8, 64),
                              (1, 2560, 10240, 8, 128),
                              (64, 10240, 2560, 8, 0), (65, 10240, 2560, 4, 0),
                              (16, 10240, 2560, 4, 0), (64, 10240, 2560, 4, 0),
                              (9, 640, 2560, 4, 0),
                              (257, 2560, 10240, 8, 64), (4096, 10240, 2560, 8, 0),
                              (1, 10240, 2560, 8, 0), (8, 512, 4096, 8, 0),
                              (64, 512, 128, 4, 0), (0, 512, 1024, 8, 0)]:
        assert cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs) == \
            cider.cider_linear_workspace_bytes(M, K), (M, N, K, bits, gs)


def test_set_path():
    assert cider.cider_set_path(2) == 0
    assert cider.cider_set_path(1) == 2
    assert cider.cider_set_path(7) == -1
    assert cider.cider_set_path(0) == 1


def _gemm(**kw):
    a = dict(xq=P, s_tok=P2, wq=P3, s_w=P4, M=16, N=128, K=256, group_size=0, y_f16=P, check=False)
    a.update(kw)
    return cider.cider_w8a8_gemm(a["xq"], a["s_tok"], a["wq"], a["s_w"], a["M"], a["N"], a["K"],
                                 a["group_size"], a["y_f16"], stream=0, check=False)


def test_gemm_argument_codes():
    assert _gemm() == cider.CIDER_ERR_NO_DEVICE
    assert _gemm(M=-1) == cider.CIDER_ERR_INVALID_ARG
    assert _gemm(K=0) == cider.CIDER_ERR_INVALID_ARG
    assert _gemm(group_size=32) == cider.CIDER_ERR_INVALID_ARG
    assert _gemm(K=96) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(N=100) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(K=192, group_size=128) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(K=133248) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(xq=None) == cider.CIDER_ERR_INVALID_ARG
    assert _gemm(s_w=None) == cider.CIDER_ERR_INVALID_ARG
    assert _gemm(xq=BAD) == cider.CIDER_ERR_MISALIGNED
    assert _gemm(y_f16=BAD) == cider.CIDER_ERR_MISALIGNED
    # empty problems are a no-op that needs neither pointers nor a device
    assert _gemm(M=0, xq=None, wq=None, y_f16=None) == cider.CIDER_OK
    assert _gemm(N=0, xq=None) == cider.CIDER_OK


def test_w4a8_argument_codes():
    f = cider.cider_w4a8_gemm
    assert f(P, P2, P3, P4, 8, 64, 128, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, P2, P3, P4, 8, 64, 128, 64, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, P2, P3, P4, 8, 64, 128, 128, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, P2, P3, P4, 8, 64, 128, 32, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert f(P, P2, P3, P4, 8, 64, 192, 128, P, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    g = cider.cider_w4a8_gemm_i32
    assert g(P, P3, 8, 64, 128, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert g(P, BAD, 8, 64, 128, 0, P, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED


def test_i32_hooks_need_no_scales():
    f = cider.cider_w8a8_gemm_i32
    assert f(P, P3, 8, 64, 128, 64, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, None, 8, 64, 128, 0, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG


def test_quantize_argument_codes():
    qa = cider.cider_quantize_act
    assert qa(P, 4, 256, 256, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qa(P, 4, 256, 128, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qa(P, 4, 256, 260, P2, P3, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    assert qa(P, 4, 200, 256, P2, P3, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert qa(P, 0, 256, 256, None, None, stream=0, check=False) == cider.CIDER_OK
    qw = cider.cider_quantize_weight
    assert qw(P, 64, 256, 8, 0, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qw(P, 64, 256, 8, 128, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qw(P, 64, 256, 4, 64, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qw(P, 64, 256, 4, 96, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qw(P, 64, 256, 6, 0, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qw(P, 64, 320, 8, 128, P2, P3, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE


def test_quantize_weight_clipped_argument_codes():
    qc = cider.cider_quantize_weight_clipped
    assert qc(P, 64, 256, 8, 0, 99.9, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qc(P, 64, 256, 4, 128, 100.0, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    for p in (0.0, -1.0, 100.5, float("nan"), float("inf")):
        assert qc(P, 64, 256, 8, 0, p, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qc(P, 64, 256, 8, 96, 99.9, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qc(P, 64, 320, 8, 128, 99.9, P2, P3, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert qc(BAD, 64, 256, 8, 0, 99.9, P2, P3, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    assert qc(P, 0, 256, 8, 0, 99.9, None, None, stream=0, check=False) == cider.CIDER_OK


def test_dtype_and_smoothing_argument_codes():
    D16, B16 = cider.CIDER_DTYPE_F16, cider.CIDER_DTYPE_BF16
    qa = cider.cider_quantize_act_ex
    assert qa(P, B16, 4, 256, 256, P4, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qa(P, D16, 4, 256, 256, None, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qa(P, 2, 4, 256, 256, None, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert qa(P, B16, 4, 256, 256, BAD, P2, P3, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    qw = cider.cider_quantize_weight_ex
    assert qw(P, B16, 64, 256, 4, 64, 99.9, P2, P3, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert qw(P, 3, 64, 256, 8, 0, 100.0, P2, P3, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    fw = cider.cider_smooth_fold_weight
    assert fw(P, B16, 64, 256, P4, P2, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert fw(P, D16, 64, 252, P4, P2, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert fw(P, D16, 64, 256, None, P2, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert fw(P, D16, 64, 256, BAD, P2, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    assert fw(P, 5, 64, 256, P4, P2, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    ge = cider.cider_gemm_ex
    assert ge(P, P2, P3, P4, 16, 128, 256, 8, 0, B16, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert ge(P, P2, P3, P4, 16, 128, 256, 4, 64, D16, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert ge(P, P2, P3, P4, 16, 128, 256, 8, 0, 2, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    le = cider.cider_linear_ex
    ws = cider.cider_linear_workspace_bytes(1, 256)
    # one bf16 token is not fused: it needs the workspace
    assert le(P, B16, 1, 256, 256, None, P3, P4, 128, 8, 0, D16, None, 0, P, stream=0,
              check=False) == cider.CIDER_ERR_WORKSPACE
    assert le(P, D16, 1, 256, 256, P4, P3, P4, 128, 8, 0, D16, None, 0, P, stream=0,
              check=False) == cider.CIDER_ERR_WORKSPACE
    assert le(P, B16, 1, 256, 256, P4, P3, P4, 128, 8, 0, B16, P2, ws, P, stream=0,
              check=False) == cider.CIDER_ERR_NO_DEVICE
    assert le(P, 7, 1, 256, 256, None, P3, P4, 128, 8, 0, D16, P2, ws, P, stream=0,
              check=False) == cider.CIDER_ERR_INVALID_ARG


def test_decode_argument_codes():
    dl = cider.cider_decode_linear
    assert dl(P, 1024, P2, P3, 100, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert dl(P, 32768, P2, P3, 64, 4, 128, 1, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert dl(P, 32768, P2, P3, 64, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert dl(P, 32832, P2, P3, 64, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert dl(P, 1000, P2, P3, 64, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert dl(P, 1024, P2, P3, 64, 8, 32, 0, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert dl(P, 1024, P2, P3, 64, 8, 0, 3, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert dl(BAD, 1024, P2, P3, 64, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    assert dl(P, 1024, P2, P3, 0, 8, 0, 0, None, stream=0, check=False) == cider.CIDER_OK


def test_linear_argument_codes():
    f = cider.cider_w8a8_linear
    ws = cider.cider_linear_workspace_bytes(16, 256)
    assert f(P, 16, 256, 256, P2, P3, 128, 0, P4, ws, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, 16, 256, 256, P2, P3, 128, 0, P4, ws - 1, P, stream=0, check=False) == cider.CIDER_ERR_WORKSPACE
    assert f(P, 16, 256, 256, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_WORKSPACE
    assert f(P, 16, 256, 200, P2, P3, 128, 0, P4, ws, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    # up to 8 fp16 tokens on the matrix-vector path: quantization fused into
    # the matrix-vector kernel, no workspace needed
    assert f(P, 1, 256, 256, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, 8, 256, 264, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    # past the matrix-vector range (M * K > 65536, or M > 4 with int4 weights)
    # the workspace is required
    assert f(P, 8, 8256, 8256, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_WORKSPACE
    assert f(P, 8, 8192, 8192, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    # a row stride that puts the last token 2 GiB or more past the first (the
    # fused kernel's 32-bit buffer offsets would wrap) leaves the fused path:
    # the tokens are quantized into the workspace instead
    big = 2 ** 29 + 2 ** 28                               # ((M - 1) * ldx + K) * 2 >= 2^31 at M = 3
    assert ((3 - 1) * big + 256) * 2 >= 2 ** 31 and ((2 - 1) * big + 256) * 2 < 2 ** 31
    assert f(P, 2, 256, big, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, 3, 256, big, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_WORKSPACE
    ws3 = cider.cider_linear_workspace_bytes(3, 256)
    assert f(P, 3, 256, big, P2, P3, 128, 0, P4, ws3, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    f4 = cider.cider_w4a8_linear
    assert f4(P, 4, 256, 256, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f4(P, 5, 256, 256, P2, P3, 128, 0, None, 0, P, stream=0, check=False) == cider.CIDER_ERR_WORKSPACE


def test_forced_gemv_range():
    assert cider.cider_set_path(cider.PATH_GEMV) == 0
    assert _gemm(M=8, K=4096) == cider.CIDER_ERR_NO_DEVICE
    assert _gemm(M=9) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(M=2, K=32768 - 64 + 64 * 256) == cider.CIDER_ERR_UNSUPPORTED_SHAPE
    assert _gemm(M=8, K=8192) == cider.CIDER_ERR_NO_DEVICE          # M * K = 65536
    assert _gemm(M=8, K=8192 + 64) == cider.CIDER_ERR_UNSUPPORTED_SHAPE


def test_raises_with_check():
    with pytest.raises(cider.CiderError):
        cider.cider_w8a8_gemm(P, P2, P3, P4, 4, 64, 96, 0, P, stream=0)


def test_linear_noalloc_argument_codes():
    """The no-allocation linear call: the same argument checks as
    cider_linear_ex, no workspace argument, and a clear status for calls
    whose workspace would not fit the static array."""
    f = cider.cider_linear_ex_noalloc
    lim = cider.CIDER_NOALLOC_SCRATCH_BYTES
    assert f(P, 0, 16, 256, 256, None, P2, P3, 128, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, 0, 16, 256, 200, None, P2, P3, 128, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert f(BAD, 0, 16, 256, 256, None, P2, P3, 128, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_MISALIGNED
    assert f(P, 2, 16, 256, 256, None, P2, P3, 128, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    assert f(P, 0, 16, 256, 256, None, P2, P3, 128, 8, 32, 0, P, stream=0, check=False) == cider.CIDER_ERR_INVALID_ARG
    # the largest token count whose activations and scales fit, and one more
    K = 10240
    M = 1
    while cider.cider_linear_workspace_bytes(M + 1, K) <= lim:
        M += 1
    assert cider.cider_linear_workspace_bytes(M, K) <= lim < cider.cider_linear_workspace_bytes(M + 1, K)
    assert f(P, 0, M, K, K, None, P2, P3, 2560, 8, 64, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert f(P, 0, M + 1, K, K, None, P2, P3, 2560, 8, 64, 0, P, stream=0, check=False) == cider.CIDER_ERR_SCRATCH_LIMIT
    # a fused one-token call needs no workspace at any size
    assert f(P, 0, 1, 65536, 65536, None, P2, P3, 128, 8, 0, 0, P, stream=0, check=False) == cider.CIDER_ERR_NO_DEVICE
    assert cider.cider_status_str(cider.CIDER_ERR_SCRATCH_LIMIT) != "unknown status"
