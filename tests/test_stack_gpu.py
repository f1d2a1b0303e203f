"""GPU parity of the layer at model scale: the 36-layer, 4096-token stack of
8B-class decoder GEMMs (QKV, O, gate+up, down; W8A8 per channel) chained
through the activation row stride exactly as the benchmark runs it.

Each GEMM of layers 0 and 35 is checked against the oracle on the fp16 input
the GPU actually consumed (so fp16 rounding drift along the chain does not
compound into the comparison):
  * weight codes and scales of those layers: bit-exact;
  * quantized activations and token scales of each GEMM input, read in place
    through its row stride: every row, bit-exact;
  * GEMM outputs: sampled rows within |d| <= 1e-3 + 2^-10 |ref| of the
    oracle, and every output within the same bound of the exact product of the
    oracle's codes and scales;
  * the final activations after 36 layers: finite."""
import numpy as np
import pytest

import bench
import synth_inputs as si
import w4a8_quantized_linear_amd as cider
from oracle.oracle import get as get_oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CHECK_LAYERS = (0, si.DECODER_LAYERS - 1)


@pytest.fixture(scope="module")
def stack_run():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert cider.cider_is_available(), "libcider.so reports no usable gfx950 device"
    cider.cider_set_path(cider.PATH_AUTO)
    gu.announce("drawing and quantizing the 36-layer stack")
    S = bench.DecoderStack(torch, cider, si, keep_fp16=CHECK_LAYERS)
    x0_np = si.activations(S.M, S.shapes[0][1])
    gu.announce("running the stack")
    out, caps = S.forward(gu.to_dev(x0_np), capture=CHECK_LAYERS)
    gu.sync()
    assert np.array_equal(caps[0][0], x0_np)
    yield S, out, caps
    del S, out
    torch.cuda.empty_cache()


def test_stack_output_finite(stack_run):
    _, out, _ = stack_run
    assert bool(out.isfinite().all().item()), "stack output must stay finite"


@pytest.mark.parametrize("layer", CHECK_LAYERS)
@pytest.mark.parametrize("j", range(len(si.DECODER_LAYER)))
def test_stack_gemm_matches_oracle(stack_run, layer, j):
    S, _, caps = stack_run
    orc = get_oracle()
    N, K = S.shapes[j]
    src = caps[layer][j]              # the buffer GEMM j reads: its first K columns
    ldx = src.shape[1]
    x = np.ascontiguousarray(src[:, :K])

    w = S.fp16[(layer, j)]
    wq_ref, sw_ref = orc.quantize_weight(w, 8, 0)
    wq, sw = S.weights[layer][j]
    assert np.array_equal(gu.to_host(sw), sw_ref), "weight scales"
    assert np.array_equal(gu.to_host(wq), wq_ref), "weight codes"

    rq, rs = orc.quantize_act(x)
    xq, st = gu.quantize_act_gpu(gu.to_dev(src), S.M, K, ldx)
    assert np.array_equal(gu.to_host(st), rs), "token scales"
    assert np.array_equal(gu.to_host(xq), rq), "activation codes"

    rows = np.array(sorted({0, 1, 255, 256, 2047, S.M - 1} |
                           set(np.random.default_rng([layer, j]).integers(0, S.M, 8).tolist())))
    ref = orc.dequant(orc.gemm_acc(rq[rows], wq_ref, 8, 0), rs[rows], sw_ref)
    gu.assert_f16_close(caps[layer][j + 1][rows], ref, "layer %d GEMM %d" % (layer, j))
    gu.assert_every_output(gu.to_dev(caps[layer][j + 1]), rq, rs, wq_ref, sw_ref, 0,
                           "layer %d GEMM %d" % (layer, j))
