"""GPU parity of the few-token linear call on the matrix-vector path: fp16
tokens (M <= 8, M * K <= 65536, any row stride) quantized inside the
matrix-vector kernel.  Checked against the oracle's whole layer (fp16 / bf16
tolerance) and, bit for bit, against the two-kernel path on the same inputs
(quantize kernel, then the matrix-vector product of the int8 tokens).
Shapes include K = 64 (a wavefront's chunks then span several tokens, so the
per-token maxima and code sums take the per-lane route) and M * K = 65536."""
import numpy as np
import pytest

import synth_inputs as si
import w4a8_quantized_linear_amd as cider
from oracle.oracle import get as get_oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MODES = [(8, 0), (8, 64), (8, 128), (4, 0), (4, 64), (4, 128)]
MODE_IDS = ["w8a8_pc", "w8a8_pg64", "w8a8_pg128", "w4a8_pc", "w4a8_pg64", "w4a8_pg128"]
SHAPES = [(2, 512, 2560, 2560), (3, 320, 1024, 1088), (5, 640, 64, 64), (8, 128, 4096, 4096),
          (7, 2560, 4096, 4160), (4, 10240, 2560, 2560), (8, 64, 64, 72), (6, 192, 5120, 5120),
          (4, 640, 10240, 10240), (6, 320, 10240, 10304), (8, 256, 8192, 8192),
          (1, 192, 40960, 40960), (1, 512, 32768, 32768)]


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


@pytest.mark.parametrize("y_dtype", [0, 1])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K,ldx", SHAPES)
def test_fused_tokens(M, N, K, ldx, bits, gs, y_dtype):
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    import torch
    assert M * K <= 65536
    cider.cider_set_path(cider.PATH_GEMV)  # the matrix-vector kernel at every shape here
    orc = get_oracle()
    x = si.activations(M, ldx, seed=M * 7 + K)
    x[M // 2, : K // 2] = 0  # a half-zero token
    xb = x.view(np.uint16)
    w = si.weights(N, K, seed=N + K)
    wq, sw = orc.quantize_weight(w, bits, gs)
    xd, wqd, swd = gu.bits_to_dev(xb), gu.to_dev(wq), gu.to_dev(sw)
    y = gu.empty((M, N), torch.int16)
    # the workspace is not needed on this path: none is given
    cider.cider_linear_ex(xd, 0, M, K, ldx, None, wqd, swd, N, bits, gs, y_dtype, None, 0, y)
    got = gu.bits_to_host(y)
    ref, _, _ = orc.linear_ex(xb, 0, wq, sw, bits, gs, K=K, y_dtype=y_dtype)
    gu.assert_out_close(got, ref, y_dtype, "fused M=%d N=%d K=%d" % (M, N, K))
    # the two-kernel path: int8 tokens from the quantize kernel, then the
    # matrix-vector product (forced) with the same output type
    xq = gu.empty((M, K), torch.int8)
    st = gu.empty((M,), torch.float32)
    cider.cider_quantize_act(xd, M, K, ldx, xq, st)
    y2 = gu.empty((M, N), torch.int16)
    cider.cider_set_path(cider.PATH_GEMV)
    cider.cider_gemm_ex(xq, st, wqd, swd, M, N, K, bits, gs, y_dtype, y2)
    cider.cider_set_path(cider.PATH_AUTO)
    assert np.array_equal(gu.bits_to_host(y2), got)
