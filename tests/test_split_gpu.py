"""GPU parity of the split-K product: linear calls of few tokens given the
workspace of cider_linear_workspace_bytes_ex split K over several workgroups
per output tile (per group up to 256 tokens, int4 per channel up to 64) and
reduce the partial sums in the last one.  Shapes the library does not split
run through the same calls and are checked the same way.

Checked against the oracle's whole layer (fp16 / bf16 tolerance), against
the unsplit call on the same inputs (per channel bit-identical: the int32
partial sums add exactly), with the workspace filled with garbage first (the
counters must be cleared by the call itself and every partial written), and
across consecutive calls that share one workspace."""
import numpy as np
import pytest

import synth_inputs as si
import w4a8_quantized_linear_amd as cider
from oracle.oracle import get as get_oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MODES = [(8, 0), (8, 64), (8, 128), (4, 0), (4, 64), (4, 128)]
MODE_IDS = ["w8a8_pc", "w8a8_pg64", "w8a8_pg128", "w4a8_pc", "w4a8_pg64", "w4a8_pg128"]
# token counts on both sides of the 64 / 128-token tiles, ragged in M; up to
# 32 tokens the few-token kernel takes the call unsplit (K = 320 / 192: K not
# a multiple of its 128-value unit, so those split); K from one split unit
# per split up to long rows
SHAPES = [(9, 640, 2560), (16, 512, 1024), (32, 192, 512), (20, 256, 320), (30, 128, 192),
          (37, 2560, 2560), (64, 1024, 4096), (100, 320, 1024), (128, 2560, 2560),
          (128, 64, 10240), (200, 320, 1024), (256, 640, 2048)]


def _splits(M, K, bits, gs):
    """Where the library splits: per group from 33 to 256 tokens, and up to 32
    where the few-token kernel does not take the shape (K not a multiple of
    128 int8 / 256 int4 values); per channel never (measured slower)."""
    few = M <= 32 and K % (128 if bits == 8 else 256) == 0
    return gs != 0 and M <= 256 and not few


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert cider.cider_is_available(), "libcider.so reports no usable gfx950 device"
    cider.cider_set_path(cider.PATH_AUTO)
    yield


@pytest.fixture(autouse=True)
def _announce(request):
    gu.announce(request.node.nodeid)
    yield


def _garbage_workspace(nbytes):
    import torch
    ws = gu.empty((max(nbytes, 16),), torch.uint8)
    ws.fill_(0xA5)
    return ws


def _linear(xb, x_dtype, M, K, wq, sw, N, bits, gs, y_dtype, ws, ws_bytes):
    import torch
    y = gu.empty((M, N), torch.int16)
    cider.cider_linear_ex(xb, x_dtype, M, K, K, None, wq, sw, N, bits, gs, y_dtype, ws, ws_bytes, y)
    return gu.bits_to_host(y)


@pytest.mark.parametrize("y_dtype", [0, 1])
@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_split_linear(M, N, K, bits, gs, y_dtype):
    if gs and K % gs:
        pytest.skip("K not a multiple of the group size")
    orc = get_oracle()
    base = cider.cider_linear_workspace_bytes(M, K)
    ex = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
    assert (ex > base) == _splits(M, K, bits, gs)
    x = si.activations(M, K, seed=M + K)
    xb = x.view(np.uint16)
    w = si.weights(N, K, seed=N)
    wq, sw = orc.quantize_weight(w, bits, gs)
    xd, wqd, swd = gu.bits_to_dev(xb), gu.to_dev(wq), gu.to_dev(sw)
    ws = _garbage_workspace(ex)
    y = _linear(xd, 0, M, K, wqd, swd, N, bits, gs, y_dtype, ws, ex)
    ref, _, _ = orc.linear_ex(xb, 0, wq, sw, bits, gs, K=K, y_dtype=y_dtype)
    gu.assert_out_close(y, ref, y_dtype, "split M=%d N=%d K=%d" % (M, N, K))
    # the same call again on the used workspace: identical bits
    y2 = _linear(xd, 0, M, K, wqd, swd, N, bits, gs, y_dtype, ws, ex)
    assert np.array_equal(y, y2)
    if gs == 0:
        y_unsplit = _linear(xd, 0, M, K, wqd, swd, N, bits, gs, y_dtype, _garbage_workspace(base), base)
        assert np.array_equal(y, y_unsplit), "per channel the split sum is exact"


@pytest.mark.parametrize("bits,gs", MODES, ids=MODE_IDS)
def test_split_consecutive_calls_share_workspace(bits, gs):
    """A large call, then a smaller one and one of another shape, through one
    workspace sized for the largest: each against the oracle."""
    orc = get_oracle()
    K = 2048
    calls = [(128, 1280), (16, 1280), (50, 640), (128, 1280)]
    size = max(cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs) for M, N in calls)
    ws = _garbage_workspace(size)
    w = si.weights(1280, K, seed=3)
    wq, sw = orc.quantize_weight(w, bits, gs)
    for i, (M, N) in enumerate(calls):
        x = si.activations(M, K, seed=10 + i)
        xb = x.view(np.uint16)
        G = 1 if gs == 0 else K // gs
        wq_n = wq[:N]
        sw_n = sw[:N] if gs == 0 else sw.reshape(1280, G)[:N]
        y = _linear(gu.bits_to_dev(xb), 0, M, K, gu.to_dev(np.ascontiguousarray(wq_n)),
                    gu.to_dev(np.ascontiguousarray(sw_n)), N, bits, gs, 0, ws, size)
        ref, _, _ = orc.linear_ex(xb, 0, wq_n, sw_n, bits, gs, K=K, y_dtype=0)
        gu.assert_out_close(y, ref, 0, "call %d M=%d N=%d" % (i, M, N))


def test_split_not_used_past_its_range_or_for_one_token():
    """Shapes the split does not serve (per channel, past 256 tokens, and the
    few-token kernel's shapes up to 32) need no extra workspace."""
    for M, bits, gs in ((257, 8, 64), (65, 4, 0), (16, 8, 0), (1, 8, 64), (32, 8, 64), (9, 4, 128)):
        assert cider.cider_linear_workspace_bytes_ex(M, 2560, 2560, bits, gs) == \
            cider.cider_linear_workspace_bytes(M, 2560)


@pytest.mark.parametrize("bits,gs,M,N,K", [(8, 64, 64, 640, 2048), (4, 0, 32, 1280, 2560),
                                           (8, 0, 1, 2560, 2560), (4, 128, 200, 320, 1024),
                                           (8, 0, 300, 640, 1024)])
def test_linear_in_hip_graph(bits, gs, M, N, K):
    """The linear call captured into a HIP graph (its tile counters are
    cleared by the quantize kernel, not by a memset node) and replayed several
    times with the program's own eager work and synchronizations in between:
    every replay equals the eager result bit for bit."""
    import torch
    orc = get_oracle()
    x = si.activations(M, K, seed=7)
    w = si.weights(N, K, seed=8)
    wq, sw = orc.quantize_weight(w, bits, gs)
    xd, wqd, swd = gu.bits_to_dev(x.view(np.uint16)), gu.to_dev(wq), gu.to_dev(sw)
    size = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
    ws = _garbage_workspace(size)
    y = gu.empty((M, N), torch.int16)
    f = cider.cider_w8a8_linear if bits == 8 else cider.cider_w4a8_linear

    def call():
        f(xd, M, K, K, wqd, swd, N, gs, None if M == 1 else ws, 0 if M == 1 else size, y)

    call()
    gu.sync()
    eager = gu.bits_to_host(y).copy()
    ref, _, _ = orc.linear_ex(x.view(np.uint16), 0, wq, sw, bits, gs, K=K, y_dtype=0)
    gu.assert_out_close(eager, ref, 0, "eager M=%d" % M)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        call()  # warm on the capture stream
        with torch.cuda.graph(g, stream=stream):
            call()
    torch.cuda.current_stream().wait_stream(stream)
    gu.sync()
    for r in range(4):
        y.zero_()
        ws.fill_(0x5A)  # the program's own eager work between replays
        gu.sync()
        g.replay()
        gu.sync()
        assert np.array_equal(gu.bits_to_host(y), eager), "replay %d" % r
