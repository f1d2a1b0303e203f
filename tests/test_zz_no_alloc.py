"""The no-allocation linear call (cider_linear_ex_noalloc) against the
workspace call it mirrors (cider_linear_ex given the split workspace size),
through the C ABI: two calls in a row on the static scratch array, the
second on a smaller input, each compared bit for bit with the workspace
call and, on sampled rows, with the oracle within the output tolerance."""
import numpy as np
import pytest

import synth_inputs as si
import w4a8_quantized_linear_amd as cider
from oracle.oracle import get as get_oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert cider.cider_is_available(), "libcider.so reports no usable gfx950 device"
    cider.cider_set_path(cider.PATH_AUTO)
    yield


def _one(M, N, K, bits, gs, x_dtype, y_dtype, smooth, seed):
    """One call of each entry point on the same inputs; returns both outputs
    (uint16 patterns), the inputs, and the oracle's sampled rows."""
    import torch
    orc = get_oracle()
    x = si.activations(M, K, seed=seed).astype(np.float32)
    xb = gu.bf16_bits(x) if x_dtype == 1 else x.astype(np.float16).view(np.uint16)
    w = si.weights(N, K, seed=seed)
    wq, sw = orc.quantize_weight(w, bits, gs)
    sm = np.random.default_rng([seed, 4]).uniform(0.5, 4.0, K).astype(np.float32) if smooth else None
    xd, wqd, swd = gu.bits_to_dev(xb), gu.to_dev(wq), gu.to_dev(sw)
    smd = gu.to_dev(sm) if smooth else None
    ws_bytes = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
    assert ws_bytes <= cider.CIDER_NOALLOC_SCRATCH_BYTES
    ws = gu.empty((max(ws_bytes, 16),), torch.uint8)
    ws.fill_(0xA5)
    y_ref = gu.empty((M, N), torch.int16)
    y_new = gu.empty((M, N), torch.int16)
    y_new.fill_(0x5A5A)
    cider.cider_linear_ex(xd, x_dtype, M, K, K, smd, wqd, swd, N, bits, gs, y_dtype, ws, ws_bytes,
                          y_ref)
    cider.cider_linear_ex_noalloc(xd, x_dtype, M, K, K, smd, wqd, swd, N, bits, gs, y_dtype, y_new)
    gu.sync()
    rows = np.unique(np.array([0, min(1, M - 1), M // 2, M - 1]))
    ref, _, _ = orc.linear_ex(np.ascontiguousarray(xb[rows]), x_dtype, wq, sw, bits, gs, K=K,
                              smooth=sm, y_dtype=y_dtype)
    return gu.bits_to_host(y_ref), gu.bits_to_host(y_new), rows, ref


CASES = [
    # (first call, second call): (M, N, K, bits, gs, x_dtype, y_dtype, smooth)
    ((4096, 10240, 2560, 8, 0, 0, 0, False), (64, 512, 1024, 8, 0, 0, 0, False)),
    ((128, 2560, 10240, 8, 64, 0, 0, False), (16, 2560, 10240, 8, 64, 0, 0, False)),
    ((64, 10240, 2560, 4, 0, 0, 0, False), (9, 640, 2560, 4, 0, 0, 0, False)),
    ((130, 640, 2560, 8, 128, 1, 1, True), (33, 640, 2560, 8, 128, 1, 1, True)),
    ((256, 2560, 10240, 4, 128, 0, 1, False), (100, 2560, 10240, 4, 128, 0, 1, False)),
    ((1, 10240, 2560, 8, 0, 0, 0, False), (1, 512, 1024, 4, 0, 0, 0, False)),
]


@pytest.mark.parametrize("first,second", CASES,
                         ids=["pc_4096_then_64", "pg64_split_128_then_16", "w4pc_split_64_then_9",
                              "bf16_smooth_pg128_130_then_33", "w4pg128_256_then_100",
                              "one_token_then_one_token"])
def test_noalloc_matches_workspace_call(first, second):
    for i, case in enumerate((first, second)):
        M, N, K, bits, gs, x_dt, y_dt, smooth = case
        gu.announce("noalloc call %d: M=%d N=%d K=%d bits=%d gs=%d x=%d y=%d smooth=%s"
                    % (i + 1, M, N, K, bits, gs, x_dt, y_dt, smooth))
        y_ref, y_new, rows, ref = _one(M, N, K, bits, gs, x_dt, y_dt, smooth, seed=M + N + i)
        assert np.array_equal(y_new, y_ref), "call %d differs from the workspace call" % (i + 1)
        gu.assert_out_close(y_new[rows], ref, y_dt, "call %d vs the oracle" % (i + 1))
