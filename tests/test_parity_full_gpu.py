"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the whole layer through cider_*_linear: per-token quantize
into the workspace, then the product kernel chosen for that M).

The oracle cannot afford every output at these sizes, so:
  * quantized activations and token scales: every row, bit-exact;
  * int32 accumulators (the _i32 hooks, same tiles as the product): sampled
    rows at tile boundaries, the ragged end and a few seeded random rows,
    bit-exact against the oracle's integer product of those rows;
  * fp16 outputs of the linear call: the same sampled rows, within
    |d| <= 1e-3 + 2^-10 |ref|; and every output against the exact product of
    the oracle's codes and scales (float64 sums on the device's dense
    product, rounded once to fp16), with the same tolerance;
  * for every row, a property that holds at any size: the all-zero token
    planted in row 3 gives exactly zero outputs.
Per-group int32 accumulators are [M, N, K/gs]; they are checked at M = 520
(the large-tile configuration, 0.85 GB) instead of M = 4096 (6.7 GB)."""
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


@pytest.fixture(autouse=True)
def _announce(request):
    gu.announce(request.node.nodeid)
    yield


def sample_rows(M, seed=0):
    """Tile edges of both product configurations (64- and 256-token tiles),
    the ragged end and seeded random rows."""
    edges = [0, 1, 2, 3, 63, 64, 255, 256, 257, 511, 512, 1023, 1024, 2047, 2048, 4095, 4096,
             6143, 8191]
    rng = np.random.default_rng([seed, 9, M])
    rows = set(r for r in edges if r < M) | {M - 2, M - 1} | set(rng.integers(0, M, 6).tolist())
    return np.array(sorted(rows))


FULL = [("w8a8_pc", 8, 0, 10240, 2560, 128), ("w8a8_pc", 8, 0, 10240, 2560, 1024),
        ("w8a8_pc", 8, 0, 10240, 2560, 4096), ("w8a8_pc", 8, 0, 10240, 2560, 8192),
        ("w8a8_pg64", 8, 64, 2560, 10240, 128), ("w8a8_pg128", 8, 128, 2560, 10240, 1024),
        ("w4a8_pc", 4, 0, 10240, 2560, 128), ("w4a8_pc", 4, 0, 10240, 2560, 2048),
        ("w8a8_pg64", 8, 64, 2560, 10240, 4096), ("w8a8_pg128", 8, 128, 2560, 10240, 4096),
        ("w4a8_pc", 4, 0, 10240, 2560, 4096), ("w4a8_pc", 4, 0, 10240, 2560, 8192),
        ("w4a8_pg64", 4, 64, 2560, 10240, 128), ("w4a8_pg128", 4, 128, 2560, 10240, 1024),
        ("w4a8_pg64", 4, 64, 2560, 10240, 4096), ("w4a8_pg128", 4, 128, 2560, 10240, 8192),
        ("w8a8_pg64", 8, 64, 2560, 10240, 1024), ("w8a8_pg64", 8, 64, 2560, 10240, 8192),
        ("w8a8_pg128", 8, 128, 2560, 10240, 128), ("w8a8_pg128", 8, 128, 2560, 10240, 8192),
        ("w4a8_pc", 4, 0, 10240, 2560, 1024)]


@pytest.mark.parametrize("name,bits,gs,N,K,M", FULL, ids=["%s_M%d" % (c[0], c[5]) for c in FULL])
def test_full_size_sampled(name, bits, gs, N, K, M):
    import torch
    orc = get_oracle()
    x = si.activations(M, K)
    x[3] = 0  # an all-zero token
    w = si.weights(N, K)
    wq, sw = orc.quantize_weight(w, bits, gs)
    xd, wqd, swd = gu.to_dev(x), gu.to_dev(wq), gu.to_dev(sw)

    # every row of the quantized activations
    rq, rs = orc.quantize_act(x)
    xq, st = gu.quantize_act_gpu(xd, M, K, K)
    assert np.array_equal(gu.to_host(st), rs)
    assert np.array_equal(gu.to_host(xq), rq)

    rows = sample_rows(M)
    ref_acc = orc.gemm_acc(rq[rows], wq, bits, gs)
    ref_y = orc.dequant(ref_acc, rs[rows], sw)

    # the whole layer, as timed
    yd = gu.linear_gpu(xd, M, K, K, wqd, swd, N, bits, gs)
    y = gu.to_host(yd)
    gu.assert_f16_close(y[rows], ref_y, "%s M=%d sampled rows" % (name, M))
    # every output against the exact product of the oracle's codes
    gu.assert_every_output(yd, rq, rs, wq if bits == 8 else gu.unpack_int4(wq), sw, gs,
                           "%s M=%d" % (name, M))
    assert not np.any(y[3]), "the zero token must give zero outputs"
    assert np.all(np.isfinite(y.astype(np.float32)))

    # int32 accumulators on the same tiles
    if gs == 0:
        acc = gu.to_host(gu.gemm_i32_gpu(xq, wqd, M, N, K, bits, gs))
        assert np.array_equal(acc[rows], ref_acc)
        del acc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gs", [64, 128])
def test_per_group_i32_large_tiles(gs):
    """Per-group int32 accumulators [M, N, K/gs] at M = 520 (the 256-token
    tile configuration, with a ragged last tile), N = 2560, K = 10240."""
    import torch
    orc = get_oracle()
    M, N, K = 520, 2560, 10240
    x = si.activations(M, K)
    w = si.weights(N, K)
    wq, sw = orc.quantize_weight(w, 8, gs)
    rq, rs = orc.quantize_act(x)
    acc = gu.to_host(gu.gemm_i32_gpu(gu.to_dev(rq), gu.to_dev(wq), M, N, K, 8, gs))
    rows = sample_rows(M)
    assert np.array_equal(acc[rows], orc.gemm_acc(rq[rows], wq, 8, gs))
    del acc
    torch.cuda.empty_cache()
