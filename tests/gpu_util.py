"""Helpers for the GPU parity tests: device copies, the tolerance check and
running the layer through the C ABI.  Imports torch lazily."""
from __future__ import annotations

import sys

import numpy as np

import w4a8_quantized_linear_amd as cider

TOL_ABS = 1e-3
TOL_REL = 2.0 ** -10


def announce(msg: str):
    sys.__stderr__.write("[gpu] %s\n" % msg)
    sys.__stderr__.flush()


def to_dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(a).cuda()


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.float16)
    return t.cpu().numpy()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def sync():
    import torch
    torch.cuda.synchronize()


def assert_f16_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """|got - ref| <= 1e-3 + 2^-10 |ref| elementwise, NaN / Inf patterns equal."""
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.array_equal(np.isnan(g), np.isnan(r)), what + ": NaN pattern differs"
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf) and np.array_equal(g[inf], r[inf]), what + ": Inf differs"
    fin = ~(np.isnan(r) | inf)
    err = np.abs(g[fin] - r[fin])
    bound = TOL_ABS + TOL_REL * np.abs(r[fin])
    bad = err > bound
    if bad.any():
        i = np.argmax(err / bound)
        raise AssertionError("%s: %d of %d outputs outside tolerance, worst |d|=%.3g at ref=%.6g "
                             "(ratio %.3g)" % (what, int(bad.sum()), bad.size, err[i], r[fin][i],
                                               err[i] / bound[i]))


def quantize_weight_gpu(w: np.ndarray, bits: int, gs: int):
    """Quantize an fp16 [N, K] weight on the GPU; returns device (wq, s_w)."""
    import torch
    N, K = w.shape
    wd = to_dev(w)
    wq = empty((N, K) if bits == 8 else (N, K // 2), torch.int8 if bits == 8 else torch.uint8)
    sw = empty((N,) if gs == 0 else (N, K // gs), torch.float32)
    cider.cider_quantize_weight(wd, N, K, bits, gs, wq, sw)
    return wq, sw


def quantize_act_gpu(xd, M, K, ldx):
    import torch
    xq = empty((M, K), torch.int8)
    st = empty((M,), torch.float32)
    cider.cider_quantize_act(xd, M, K, ldx, xq, st)
    return xq, st


def gemm_gpu(xq, st, wq, sw, M, N, K, bits, gs):
    import torch
    y = empty((M, N), torch.float16)
    f = cider.cider_w8a8_gemm if bits == 8 else cider.cider_w4a8_gemm
    f(xq, st, wq, sw, M, N, K, gs, y)
    return y


def gemm_i32_gpu(xq, wq, M, N, K, bits, gs):
    import torch
    G = 1 if gs == 0 else K // gs
    acc = empty((M, N) if gs == 0 else (M, N, G), torch.int32)
    f = cider.cider_w8a8_gemm_i32 if bits == 8 else cider.cider_w4a8_gemm_i32
    f(xq, wq, M, N, K, gs, acc)
    return acc


def linear_gpu(xd, M, K, ldx, wq, sw, N, bits, gs, split=True):
    """The linear entry point; split=True hands it the workspace that lets
    it split K (as the benchmark does), split=False the minimal one."""
    import torch
    ws_bytes = (cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs) if split
                else cider.cider_linear_workspace_bytes(M, K))
    ws = empty((max(ws_bytes, 16),), torch.uint8)
    y = empty((M, N), torch.float16)
    f = cider.cider_w8a8_linear if bits == 8 else cider.cider_w4a8_linear
    f(xd, M, K, ldx, wq, sw, N, gs, ws, ws_bytes, y)
    return y


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def unpack_int4(wq4: np.ndarray) -> np.ndarray:
    """Codes q = u - 8 of packed nibbles (low nibble = even k)."""
    lo = (wq4 & 0x0F).astype(np.int16) - 8
    hi = (wq4 >> 4).astype(np.int16) - 8
    return np.stack([lo, hi], axis=-1).reshape(wq4.shape[0], -1).astype(np.int8)


def assert_every_output(y_dev, xq: np.ndarray, s_tok: np.ndarray, wcodes: np.ndarray,
                        s_w: np.ndarray, gs: int, what: str = "", rows_per_chunk: int = 512):
    """Every output of a full-size product against the exact result of the
    oracle's codes and scales: the integer sums are formed in float64 by the
    device's dense product (exact: every partial sum is an integer below
    2^53), scaled in float64, rounded once to fp16, then compared with the
    fp16 tolerance.  A property check at sizes the oracle cannot finish; the
    sampled rows of the same tests are compared with the oracle itself."""
    import torch
    M, K = xq.shape
    N = wcodes.shape[0]
    y = to_host(y_dev)
    W = torch.from_numpy(wcodes).cuda().double()
    sw = torch.from_numpy(np.ascontiguousarray(s_w, dtype=np.float32)).cuda().double()
    st = torch.from_numpy(s_tok).cuda().double()
    G = 1 if gs == 0 else K // gs
    if gs:
        Wg = W.view(N, G, gs).permute(1, 2, 0).contiguous()          # [G, gs, N]
    for r0 in range(0, M, rows_per_chunk):
        r1 = min(M, r0 + rows_per_chunk)
        X = torch.from_numpy(xq[r0:r1]).cuda().double()
        if gs == 0:
            t = (X @ W.t().contiguous()) * sw[None, :]
        else:
            acc = torch.bmm(X.view(r1 - r0, G, gs).permute(1, 0, 2).contiguous(), Wg)  # [G, m, N]
            t = (acc * sw.t().contiguous()[:, None, :]).sum(0)
        ref = (t * st[r0:r1, None]).cpu().numpy().astype(np.float16)
        assert_f16_close(y[r0:r1], ref, "%s rows %d..%d" % (what, r0, r1))
    del W, sw, st


def bf16_bits(values) -> np.ndarray:
    """uint16 patterns of fp32 values rounded to bf16 (torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_dev(a: np.ndarray):
    """uint16 patterns onto the device (as an int16 tensor)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def bits_to_host(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == 1:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def assert_out_close(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: int, what: str = ""):
    """fp16 outputs: |d| <= 1e-3 + 2^-10 |ref|.  bf16 outputs (8 significant
    bits): within one bf16 ulp of the reference, |d| <= 1e-3 + 2^-7 |ref|."""
    if dtype == 0:
        return assert_f16_close(got_bits.view(np.float16), ref_bits.view(np.float16), what)
    g, r = bits_to_f64(got_bits, 1), bits_to_f64(ref_bits, 1)
    assert np.array_equal(np.isnan(g), np.isnan(r)), what + ": NaN pattern differs"
    fin = np.isfinite(r)
    assert np.array_equal(g[~fin & ~np.isnan(r)], r[~fin & ~np.isnan(r)]), what + ": Inf differs"
    err = np.abs(g[fin] - r[fin])
    bound = 1e-3 + 2.0 ** -7 * np.abs(r[fin])
    bad = err > bound
    assert not bad.any(), "%s: %d of %d bf16 outputs outside tolerance (worst |d|=%.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max()))
