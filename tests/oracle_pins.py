"""Pins that tie the oracle to facts outside itself.

Each ``pin_*`` function takes an ``Oracle`` and raises AssertionError when the
oracle disagrees with a closed form, a hand-worked fixture, a library routine
for a special case, brute force on tiny inputs, or an invariant of the method.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutations.py``
runs them on copies of the oracle with a planted mistake and requires that at
least one pin fails for every planted mistake.

Sources (the pages print no worked example, so the pins are definitions):
  Cider README (ossradar.top repo page), 'Quantization' table: symmetric INT8
  activations per token, symmetric INT8 weights per channel or per group of
  64/128, symmetric INT4 weights with zero-point 8 packed in uint8, INT32
  accumulation, C_fp16 = C_int32 * s_act * s_weight per element.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(a):
    return np.asarray(a, dtype=np.float16)


# ----------------------------------------------------------------- fp16 ---

def pin_half_decode_exhaustive(orc):
    """All 65536 binary16 patterns widen exactly as numpy's float16 does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_double_to_half_vs_numpy(orc):
    """Rounding a double to fp16 agrees with numpy's float64 -> float16 on every
    representable value, every midpoint between neighbours (exact ties), points
    just either side of the midpoints, the overflow edge and random doubles."""
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (finite[:-1] + finite[1:]) / 2.0
    eps_lo = np.nextafter(mids, 0.0)
    eps_hi = np.nextafter(mids, np.inf)
    rng = np.random.default_rng(7)
    rand = np.exp(rng.uniform(np.log(1e-9), np.log(1e6), 20000))
    edge = np.array([65504.0, 65519.999, 65520.0, 65535.0, 65536.0, 1e9, 2.0 ** -25,
                     2.0 ** -25 * 1.0000001, 2.0 ** -24 * 1.5, 2.0 ** -14, 0.0])
    vals = np.concatenate([finite, mids, eps_lo, eps_hi, rand, edge])
    vals = np.concatenate([vals, -vals])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.double_to_half(v) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "double->half mismatch at %r" % (vals[bad[:5]],)


# ---------------------------------------------------------- quantization ---

def pin_scale_closed_forms(orc):
    """absmax 127 * 2^j gives the fp32 scale 2^j exactly (int8); absmax 7 * 2^j
    gives 2^j for int4.  One row per j, the absmax placed at a varying column."""
    js = np.arange(-12, 9)
    K = 64
    x = np.zeros((js.size, K), np.float16)
    rng = np.random.default_rng(1)
    for i, j in enumerate(js):
        x[i] = _f16(rng.uniform(-1, 1, K) * 100.0 * 2.0 ** float(j))
        x[i, (5 * i) % K] = 127.0 * 2.0 ** float(j) * (-1 if i % 2 else 1)
    _, s = orc.quantize_act(x)
    assert np.array_equal(s, (2.0 ** js).astype(np.float32)), s
    w = np.zeros((js.size, K), np.float16)
    for i, j in enumerate(js):
        w[i] = _f16(rng.uniform(-1, 1, K) * 6.0 * 2.0 ** float(j))
        w[i, (3 * i) % K] = -7.0 * 2.0 ** float(j)
    _, s4 = orc.quantize_weight(w, bits=4)
    assert np.array_equal(s4, (2.0 ** js).astype(np.float32)), s4
    _, s8 = orc.quantize_weight(x, bits=8)
    assert np.array_equal(s8, (2.0 ** js).astype(np.float32)), s8
    _, sg = orc.quantize_weight(np.concatenate([x, x[::-1]], axis=1), bits=8, group_size=K)
    assert np.array_equal(sg, np.stack([2.0 ** js, 2.0 ** js[::-1]], 1).astype(np.float32))


def _rn32(fr):
    """Round a rational to the nearest binary32 value, ties to even (normal
    range only), as an exact Fraction: the definition of a correctly rounded
    fp32 operation."""
    from fractions import Fraction
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (e - 23)            # 24-bit significand
    return sign * _rne_int(a / quantum) * quantum


def _rne_int(fr):
    """Nearest integer to a rational, ties to even."""
    import math
    fl = math.floor(fr)
    d = fr - fl
    if d * 2 < 1:
        return fl
    if d * 2 > 1:
        return fl + 1
    return fl if fl % 2 == 0 else fl + 1


def pin_quotient_exact_rational(orc):
    """Scale and codes against exact rational arithmetic: s = RN32(absmax/127)
    and q = RNE(RN32(x/s)).  Rows hold absmax a and x = a/2, whose quotient is
    within an fp32 ulp of the tie 63.5 (the case where dividing and multiplying
    by a reciprocal disagree), plus random entries; int4 weights likewise with
    7 and 3.5."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    allh = np.arange(0x0400, 0x7C00, dtype=np.uint16).view(np.float16)
    amax = rng.choice(allh[allh >= 2.0], 300, replace=False)
    K = 8
    x = np.zeros((amax.size, K), np.float16)
    x[:, 0] = amax
    x[:, 1] = (amax.astype(np.float32) / 2).astype(np.float16)   # exact (a >= 2)
    x[:, 2] = -x[:, 1]
    x[:, 3:] = (rng.uniform(-1, 1, (amax.size, K - 3)) * amax[:, None].astype(np.float64)
                ).astype(np.float16)
    for bits, qmax in ((8, 127), (4, 7)):
        if bits == 8:
            xq, s = orc.quantize_act(x)
            codes = xq.astype(np.int64)
        else:
            wq, s = orc.quantize_weight(x, bits=4)
            codes = np.empty((amax.size, K), np.int64)
            codes[:, 0::2] = (wq & 0xF).astype(np.int64) - 8
            codes[:, 1::2] = (wq >> 4).astype(np.int64) - 8
        for i in range(amax.size):
            a = Fraction(float(amax[i]))
            s_ref = _rn32(a / qmax)
            assert Fraction(float(s[i])) == s_ref, (bits, float(amax[i]))
            for k in range(K):
                q_ref = _rne_int(_rn32(Fraction(float(x[i, k])) / s_ref))
                q_ref = max(-qmax - (1 if bits == 4 else 0), min(qmax, q_ref))
                assert codes[i, k] == q_ref, (bits, float(amax[i]), float(x[i, k]))


def pin_tie_table(orc):
    """Hand-worked codes for a row with scale exactly 1 (golden fixture)."""
    g = _golden("rounding_ties.json")
    x = _f16(g["row"])[None, :]
    assert np.array_equal(x.astype(np.float64)[0], np.array(g["row"]))  # all fp16-exact
    xq, s = orc.quantize_act(x)
    assert s[0] == np.float32(g["scale"])
    assert xq[0].tolist() == g["codes_half_even"]
    assert xq[0].tolist() != g["codes_half_away_from_zero"]


def pin_weight_int8_roundtrip(orc):
    """w = q/128 with max|q| = 127 in each row (or group): scale is exactly 1/128
    and the codes come back exactly; same per group of 64 and 128."""
    rng = np.random.default_rng(2)
    N, K = 9, 256
    for gs in (0, 64, 128):
        q = rng.integers(-127, 128, size=(N, K))
        G = 1 if gs == 0 else K // gs
        L = K if gs == 0 else gs
        for n in range(N):
            for g in range(G):
                q[n, g * L + rng.integers(0, L)] = 127 if (n + g) % 2 else -127
        w = _f16(q / 128.0)
        wq, s = orc.quantize_weight(w, bits=8, group_size=gs)
        assert np.array_equal(wq.astype(np.int64), q)
        assert np.all(s == np.float32(1.0 / 128.0)) and s.size == N * G


def pin_weight_int4_roundtrip_and_packing(orc):
    """w = q/8 with max|q| = 7: scale 1/8, codes recovered, nibbles packed as
    the hand-worked fixture says; plus a random matrix unpacked by shifts."""
    g = _golden("int4_packing.json")
    w = _f16(np.array(g["q"]) / 8.0)[None, :]
    wq, s = orc.quantize_weight(w, bits=4)
    assert s[0] == np.float32(g["scale"])
    assert wq[0].tolist() == g["bytes"]
    rng = np.random.default_rng(3)
    N, K = 7, 128
    q = rng.integers(-7, 8, size=(N, K))
    q[:, 11] = 7
    wq, s = orc.quantize_weight(_f16(q / 8.0), bits=4)
    assert np.all(s == np.float32(0.125))
    lo = (wq & 0xF).astype(np.int64) - 8
    hi = (wq >> 4).astype(np.int64) - 8
    assert np.array_equal(lo, q[:, 0::2]) and np.array_equal(hi, q[:, 1::2])


def pin_weight_int4_group_roundtrip(orc):
    """int4 codes per group of 64 / 128: group g of row n holds q * 2^-(3+e)
    with max|q| = 7, so its scale is exactly 2^-(3+e) (absmax / 7) and its
    codes come back; an all-zero group has scale 0 and nibbles 8; a group
    size of K reproduces the per-channel bytes and scales."""
    rng = np.random.default_rng(12)
    N, K = 5, 512
    for gs in (64, 128):
        G = K // gs
        q = rng.integers(-7, 8, size=(N, K))
        for n in range(N):
            for g in range(G):
                q[n, g * gs + rng.integers(0, gs)] = 7 if (n + g) % 2 else -7
        e = rng.integers(0, 4, size=(N, G))
        scale = 2.0 ** -(3.0 + e)
        q[1, gs:2 * gs] = 0
        w = _f16(q * np.repeat(scale, gs, axis=1))
        wq, s = orc.quantize_weight(w, bits=4, group_size=gs)
        expect = scale.astype(np.float32)
        expect[1, 1] = 0
        assert s.shape == (N, G) and np.array_equal(s, expect), gs
        assert np.array_equal(_unpack4(wq), q), gs
        assert np.all(wq[1, gs // 2:gs] == 0x88), gs
    w = _f16(rng.standard_normal((N, K)))
    a, sa = orc.quantize_weight(w, bits=4, group_size=K)
    b, sb = orc.quantize_weight(w, bits=4)
    assert np.array_equal(a, b) and np.array_equal(sa.reshape(-1), sb)


def pin_zero_rows_and_ranges(orc):
    """All-zero row/group: scale 0, codes 0, output 0.  Codes stay in
    [-127, 127] (int8) and nibbles in [0, 15] with q in [-8, 7] (int4)."""
    x = np.zeros((3, 128), np.float16)
    x[1] = _f16(np.linspace(-90, 90, 128))
    xq, s = orc.quantize_act(x)
    assert s[0] == 0 and s[2] == 0 and not xq[0].any() and not xq[2].any()
    assert xq.min() >= -127 and xq.max() <= 127 and -127 in xq and 127 in xq
    w = _f16(np.random.default_rng(4).standard_normal((4, 128)))
    w[2, :64] = 0
    wq, sw = orc.quantize_weight(w, bits=8, group_size=64)
    assert sw[2, 0] == 0 and not wq[2, :64].any() and sw[2, 1] > 0
    wq4, sw4 = orc.quantize_weight(w, bits=4)
    u = np.concatenate([wq4 & 0xF, wq4 >> 4], axis=1)
    assert u.min() >= 0 and u.max() <= 15
    y = orc.dequant(orc.gemm_acc(xq, wq, 8, 64), s, sw)
    assert not y.astype(np.float32)[0].any() and not y.astype(np.float32)[2].any()


def pin_strided_rows(orc):
    """Quantizing the first K columns of rows with stride ldx > K equals
    quantizing the contiguous slice."""
    from synth_inputs import activations
    x = activations(5, 96)
    a, sa = orc.quantize_act(x, K=64)
    b, sb = orc.quantize_act(np.ascontiguousarray(x[:, :64]))
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


# ------------------------------------------------------------- clipping ---

def pin_percentile_vs_numpy(orc):
    """The clipping range is numpy.percentile (default linear method) of |w|
    in float64, to the bit, over rows with ties, zeros and random values, for
    several percentiles and row lengths."""
    rng = np.random.default_rng(21)
    for n in (64, 128, 1000, 2560):
        half_zero = rng.standard_normal(n)
        half_zero[: n // 2] = 0
        rows = [rng.standard_normal(n), np.round(rng.standard_normal(n) * 4) / 4, np.zeros(n),
                half_zero, 0.02 * rng.standard_normal(n)]
        for row in rows:
            h = _f16(row)
            a = np.abs(h.astype(np.float64))
            for p in (99.9, 99.0, 99.99, 50.0, 37.3, 0.1, 100.0):
                assert orc.percentile_abs(h, p) == float(np.percentile(a, p)), (n, p)


def pin_clip_100_is_absmax(orc):
    """clip_percentile = 100 reproduces plain absmax quantization in every
    weight mode, bit for bit."""
    w = _f16(np.random.default_rng(22).standard_normal((6, 256)))
    for bits, gs in ((8, 0), (8, 64), (8, 128), (4, 0), (4, 64), (4, 128)):
        a, sa = orc.quantize_weight(w, bits, gs)
        b, sb = orc.quantize_weight_clipped(w, bits, gs, 100.0)
        assert np.array_equal(a, b) and np.array_equal(sa, sb), (bits, gs)


def pin_clip_closed_forms(orc):
    """Rows whose percentile is known in closed form.  int8: |w| = k/1024,
    k = 0..1024, shuffled with random signs: the 90th percentile is 0.9, so
    s = fp32(0.9)/127 and every |w| past 0.9 + s/2 saturates at +-127.
    int4, groups of 64: |w| = k/64, k = 0..63: the 50th percentile is
    31.5/64, s = (31.5/64)/7, and the large values saturate at 7 (positive)
    and -8 (negative)."""
    rng = np.random.default_rng(23)
    k = rng.permutation(1025)
    sign = np.where(rng.integers(0, 2, 1025) == 1, 1.0, -1.0)
    w = _f16(sign * k / 1024.0)[None, :]
    wq, s = orc.quantize_weight_clipped(w, 8, 0, 90.0)
    s_exp = np.float32(np.float32(0.9) / np.float32(127.0))
    assert s[0] == s_exp
    big = np.abs(w[0].astype(np.float64)) > 0.9 + float(s_exp) / 2 + 1e-9
    assert np.array_equal(wq[0][big].astype(np.int64), (127 * sign[big]).astype(np.int64))
    assert np.all(np.abs(wq[0][~big].astype(np.int64)) <= 127)
    assert np.all(wq[0][k == 0] == 0)
    order = np.argsort(np.abs(w[0].astype(np.float64)), kind="stable")
    assert np.all(np.diff(np.abs(wq[0].astype(np.int64))[order]) >= 0)
    # int4, one group of 64 per row, two rows
    kk = np.stack([rng.permutation(64), rng.permutation(64)])
    sg = np.where(rng.integers(0, 2, (2, 64)) == 1, 1.0, -1.0)
    w4 = _f16(sg * kk / 64.0)
    wq4, s4 = orc.quantize_weight_clipped(w4, 4, 64, 50.0)
    assert np.all(s4 == np.float32(np.float32(31.5 / 64.0) / np.float32(7.0)))
    q = _unpack4(wq4)
    ratio = (sg * kk / 64.0) / float(s4[0, 0])
    assert np.array_equal(q[ratio >= 7.5], np.full(int((ratio >= 7.5).sum()), 7))
    assert np.array_equal(q[ratio <= -8.5], np.full(int((ratio <= -8.5).sum()), -8))
    assert (ratio <= -8.5).any() and (ratio >= 7.5).any()


# ------------------------------------------------- bf16 and smoothing ---

def _torch_bf16_bits(values_f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_bf16_decode_exhaustive(orc):
    """All 2^16 bf16 patterns widen to the value torch's bfloat16 type gives."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_bf16_encode(orc):
    """Rounding to bf16 agrees with torch's float32 -> bfloat16 conversion
    (round to nearest even) on fp32-exact inputs: every bf16 value, the
    midpoints between neighbours (ties), their float32 neighbours, random
    values, the overflow edge and subnormals; plus hand-worked fp64 inputs
    that fp32 cannot hold (golden fixture)."""
    rng = np.random.default_rng(31)
    b = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (b << 16).view(np.float32)
    mids = ((b << 16) + 0x8000).view(np.float32)
    xs = np.concatenate([vals, mids, np.nextafter(mids, np.float32(np.inf)),
                         np.nextafter(mids, np.float32(0)), rng.standard_normal(20000).astype(np.float32),
                         np.float32([3.3895314e38, 3.3961775e38, 3.4028235e38, 1e-40, 9.2e-41])])
    xs = np.concatenate([xs, -xs])
    ref = _torch_bf16_bits(xs)
    got = np.array([orc.double_to_bf16(float(v)) for v in xs], np.uint16)
    assert np.array_equal(got, ref)
    g = _golden("bf16_rounding.json")
    for case in g["cases"]:
        v = float.fromhex(case["value_hex"])
        assert orc.double_to_bf16(v) == int(case["bits"], 16), case


def pin_bf16_activations_match_fp16(orc):
    """Values held exactly by both types (at most 8 significant bits, within
    fp16's normal range) quantize identically from either type."""
    rng = np.random.default_rng(32)
    m = rng.integers(-255, 256, size=(6, 512)).astype(np.float64)
    e = rng.integers(-6, 4, size=(6, 512)).astype(np.float64)
    x = m * 2.0 ** e
    h = _f16(x)
    assert np.array_equal(h.astype(np.float64), x)
    bb = _torch_bf16_bits(x.astype(np.float32))
    a, sa = orc.quantize_act(h)
    b, sb = orc.quantize_act_ex(bb, 1)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    wa, wsa = orc.quantize_weight(h, 4, 64)
    wb, wsb = orc.quantize_weight_ex(bb, 1, 4, 64)
    assert np.array_equal(wa, wb) and np.array_equal(wsa, wsb)


def pin_smoothing_closed_forms(orc):
    """Smoothing divides each channel before the absmax: factors of 1 change
    nothing; power-of-two factors equal quantizing the exactly rescaled
    values; a lone outlier channel divided by its own size stops dominating
    the scale (the whole row then quantizes to 127)."""
    from synth_inputs import activations
    x = activations(5, 256, seed=7)
    a, sa = orc.quantize_act(x)
    b, sb = orc.quantize_act_ex(x, 0, smooth=np.ones(256, np.float32))
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    rng = np.random.default_rng(33)
    j = rng.integers(-2, 3, 256)
    xs = _f16(np.round(rng.standard_normal((5, 256)) * 64) / 64)
    scaled = _f16(xs.astype(np.float64) * 2.0 ** -j)
    assert np.array_equal(scaled.astype(np.float64), xs.astype(np.float64) * 2.0 ** -j)
    c, sc = orc.quantize_act_ex(xs, 0, smooth=(2.0 ** j).astype(np.float32))
    d, sd = orc.quantize_act(scaled)
    assert np.array_equal(c, d) and np.array_equal(sc, sd)
    row = np.ones((1, 64), np.float16)
    row[0, 0] = 100
    lam = np.ones(64, np.float32)
    lam[0] = 100
    q, s = orc.quantize_act_ex(row, 0, smooth=lam)
    assert np.all(q == 127) and s[0] == np.float32(1.0) / np.float32(127.0)
    q0, _ = orc.quantize_act(row)
    assert q0[0, 0] == 127 and np.all(q0[0, 1:] == 1)


def pin_smooth_fold(orc):
    """The weight fold w * smooth[k] is rounded once: power-of-two factors
    scale exactly; general fp32 factors match numpy's correctly rounded
    float64 -> float16 conversion; bf16 weights with factors whose products
    fit fp32 match torch's float32 -> bfloat16 conversion."""
    rng = np.random.default_rng(34)
    N, K = 64, 4096
    w = _f16(0.05 * rng.standard_normal((N, K)))
    j = rng.integers(0, 4, K)  # upward: no fp16 subnormal loses bits
    out = orc.smooth_fold_weight(w, 0, (2.0 ** j).astype(np.float32)).view(np.float16)
    assert np.array_equal(out.astype(np.float64), w.astype(np.float64) * 2.0 ** j)
    lam = rng.uniform(0.05, 20.0, K).astype(np.float32)
    out = orc.smooth_fold_weight(w, 0, lam)
    ref = (w.astype(np.float64) * lam.astype(np.float64)).astype(np.float16).view(np.uint16)
    assert np.array_equal(out, ref)
    wb = _torch_bf16_bits(0.05 * rng.standard_normal((N, K)))
    lam16 = (rng.integers(1, 2 ** 16, K) * 2.0 ** -12).astype(np.float32)    # 16 significant bits
    wb_val = (wb.astype(np.uint32) << 16).view(np.float32)
    prod = wb_val.astype(np.float64) * lam16.astype(np.float64)
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)  # exact in fp32
    out = orc.smooth_fold_weight(wb, 1, lam16)
    assert np.array_equal(out, _torch_bf16_bits(prod.astype(np.float32)))


def pin_bf16_output_nearest(orc):
    """bf16 outputs are the nearest bf16 values of the float64 dequant that
    the fp16 outputs are pinned on: for every output, no other bf16 value is
    closer to numpy's float64 (xq * s_tok) @ (wq * s_w)^T."""
    from synth_inputs import activations, weights
    x = activations(8, 512, seed=12)
    w = weights(40, 512, seed=12)
    for bits, gs in ((8, 0), (8, 64), (4, 128)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        yb, xq, st = orc.linear_ex(x, 0, wq, sw, bits, gs, y_dtype=1)
        codes = wq.astype(np.int64) if bits == 8 else _unpack4(wq)
        L = 512 if gs == 0 else gs
        swf = np.repeat(np.asarray(sw, np.float64).reshape(40, -1), L, axis=1)
        ref = (xq.astype(np.float64) * st.astype(np.float64)[:, None]) @ (codes * swf).T
        got = (yb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        up = (((yb.astype(np.uint32) + 1) << 16).view(np.float32)).astype(np.float64)
        dn = (((yb.astype(np.uint32) - 1) << 16).view(np.float32)).astype(np.float64)
        err = np.abs(got - ref)
        assert np.all(err <= np.abs(up - ref) * (1 + 1e-9)) and np.all(err <= np.abs(dn - ref) * (1 + 1e-9))
        assert np.array_equal(orc.dequant_ex(orc.gemm_acc(xq, wq, bits, gs), st, sw, 1), yb)
        yh, _, _ = orc.linear_ex(x, 0, wq, sw, bits, gs, y_dtype=0)
        assert np.array_equal(yh.view(np.float16), orc.linear(x, wq, sw, bits, gs)[0])


def pin_smoothing_improves_outlier_workload(orc):
    """What smoothing is for: on the outlier workload (1% of input channels
    20x larger), SmoothQuant factors lam_k = sqrt(max|X_k| / max|W_k|) with
    the weights folded bring the quantized layer much closer to the fp16
    product than plain W8A8."""
    from synth_inputs import activations, weights
    x = activations(64, 1024)
    w = weights(256, 1024)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    wq, sw = orc.quantize_weight(w, 8, 0)
    y0 = orc.linear(x, wq, sw)[0].astype(np.float64)
    ax = np.abs(x.astype(np.float64)).max(0)
    aw = np.abs(w.astype(np.float64)).max(0)
    lam = np.sqrt(ax / aw).astype(np.float32)
    wf = orc.smooth_fold_weight(w, 0, lam).view(np.float16)
    wq1, sw1 = orc.quantize_weight(wf, 8, 0)
    y1 = orc.linear_ex(x, 0, wq1, sw1, smooth=lam)[0].view(np.float16).astype(np.float64)
    e0 = np.linalg.norm(y0 - ref) / np.linalg.norm(ref)
    e1 = np.linalg.norm(y1 - ref) / np.linalg.norm(ref)
    assert e1 < 0.6 * e0, (e0, e1)


# ------------------------------------------------------ decode variant ---

def pin_decode_one_hot_and_exact(orc):
    """Decode variant, closed forms.  A one-hot x = c e_j picks one weight:
    y[n] = fp16(c * q[n, j] * s_w[n, g(j)]).  With scales that are powers of
    two and x of small dyadic values every partial sum is exact in fp64, so
    y is the exactly rounded dot product numpy computes in float64."""
    from synth_inputs import weights
    rng = np.random.default_rng(41)
    K, N = 512, 48
    w = weights(N, K, seed=41)
    for bits, gs in ((8, 0), (8, 64), (4, 0), (4, 128)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        codes = wq.astype(np.int64) if bits == 8 else _unpack4(wq)
        L = K if gs == 0 else gs
        swf = np.asarray(sw, np.float64).reshape(N, -1)
        for j in (0, 5, 200, K - 1):
            x = np.zeros(K, np.float16)
            x[j] = np.float16(1.5)
            y = orc.decode_linear(x, 0, wq, sw, bits, gs).view(np.float16)
            ref = (1.5 * codes[:, j] * swf[:, j // L]).astype(np.float16)
            assert np.array_equal(y, ref), (bits, gs, j)
    # power-of-two scales: w = q * 2^-e per row / group
    q = rng.integers(-127, 128, size=(N, K))
    q[:, 0] = 127
    e = rng.integers(6, 10, size=(N, 1))
    w2 = _f16(q * 2.0 ** -e)
    wq, sw = orc.quantize_weight(w2, 8, 0)
    assert np.array_equal(sw, (127 * 2.0 ** -e[:, 0] / 127).astype(np.float32))
    x = _f16(rng.integers(-64, 65, K) / 16.0)
    y = orc.decode_linear(x, 0, wq, sw, 8, 0).view(np.float16)
    ref = (wq.astype(np.float64) * sw.astype(np.float64)[:, None]) @ x.astype(np.float64)
    assert np.array_equal(y, ref.astype(np.float16))


def pin_decode_nearest_rational(orc):
    """Decode variant on random tiny inputs: every output is the fp16 value
    nearest to the exact rational result (Python fractions), per channel and
    per group, int8 and int4, fp16 and bf16 activations."""
    from fractions import Fraction
    from synth_inputs import activations, weights
    K, N = 128, 6
    x = activations(1, K, seed=43)[0]
    xb16 = _torch_bf16_bits(x.astype(np.float32))
    w = weights(N, K, seed=43)
    for bits, gs in ((8, 0), (8, 64), (4, 0), (4, 64)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        codes = wq.astype(np.int64) if bits == 8 else _unpack4(wq)
        L = K if gs == 0 else gs
        swf = np.asarray(sw, np.float32).reshape(N, -1)
        for xd, xbits in ((0, x.view(np.uint16)), (1, xb16)):
            xv = [Fraction(float(v)) for v in (x.astype(np.float64) if xd == 0 else
                                              (xb16.astype(np.uint32) << 16).view(np.float32))]
            y = orc.decode_linear(xbits, xd, wq, sw, bits, gs).view(np.float16)
            for n in range(N):
                exact = sum(Fraction(float(swf[n, g])) *
                            sum(xv[k] * int(codes[n, k]) for k in range(g * L, (g + 1) * L))
                            for g in range(K // L))
                got = Fraction(float(y[n]))
                up = Fraction(float(np.nextafter(y[n], np.float16(np.inf))))
                dn = Fraction(float(np.nextafter(y[n], np.float16(-np.inf))))
                assert abs(got - exact) <= abs(up - exact) and abs(got - exact) <= abs(dn - exact)


# ---------------------------------------------------------- accumulation ---

def _brute_acc(xq, wcodes, gs):
    M, K = xq.shape
    N = wcodes.shape[0]
    L = K if gs == 0 else gs
    G = K // L
    out = np.zeros((M, N, G), np.int64)
    for m in range(M):
        xr = [int(v) for v in xq[m]]
        for n in range(N):
            wr = [int(v) for v in wcodes[n]]
            for g in range(G):
                t = 0
                for k in range(g * L, (g + 1) * L):
                    t += xr[k] * wr[k]
                out[m, n, g] = t
    return out


def pin_acc_brute_force(orc):
    """int32 accumulators equal pure-Python integer dot products on tiny random
    shapes, per channel and per group (64, 128), int8 and packed int4."""
    rng = np.random.default_rng(5)
    for (M, N, K) in ((3, 5, 128), (2, 3, 256), (1, 4, 64)):
        xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        w8 = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        q4 = rng.integers(-8, 8, size=(N, K))
        w4 = ((q4[:, 0::2] + 8) | ((q4[:, 1::2] + 8) << 4)).astype(np.uint8)
        for gs in (0, 64, 128):
            if gs and K % gs:
                continue
            ref8 = _brute_acc(xq, w8.astype(np.int64), gs)
            got8 = orc.gemm_acc(xq, w8, 8, gs).reshape(ref8.shape)
            assert np.array_equal(got8, ref8), (M, N, K, gs)
            ref4 = _brute_acc(xq, q4, gs)
            got4 = orc.gemm_acc(xq, w4, 4, gs).reshape(ref4.shape)
            assert np.array_equal(got4, ref4), (M, N, K, gs, "int4")


def pin_acc_extremes(orc):
    """All-(+127) times all-(-127) reaches -K*127^2 exactly; an int4 row of -8
    codes gives -8 * sum(x); the int32 overflow bound is reported, not wrapped."""
    K = 1024
    xq = np.full((1, K), 127, np.int8)
    w = np.full((1, K), -127, np.int8)
    assert orc.gemm_acc(xq, w)[0, 0] == -K * 127 * 127
    w4 = np.zeros((1, K // 2), np.uint8)  # nibble 0 -> q = -8
    xr = np.random.default_rng(6).integers(-127, 128, size=(1, K)).astype(np.int8)
    assert orc.gemm_acc(xr, w4, 4)[0, 0] == -8 * int(xr.astype(np.int64).sum())
    Kbig = 133248  # 127^2 * Kbig > 2^31 - 1
    from oracle.oracle import OracleError
    try:
        orc.gemm_acc(np.full((1, Kbig), 127, np.int8), np.full((1, Kbig), 127, np.int8))
    except OracleError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


def pin_group_reductions(orc):
    """group_size = K reproduces per-channel; the per-group partial sums add up
    to the per-channel sum; equal group scales reduce per-group dequant to the
    per-channel one."""
    rng = np.random.default_rng(8)
    M, N, K = 4, 6, 256
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    pc = orc.gemm_acc(xq, w, 8, 0)
    assert np.array_equal(orc.gemm_acc(xq, w, 8, K)[:, :, 0], pc)
    for gs in (64, 128):
        pg = orc.gemm_acc(xq, w, 8, gs)
        assert np.array_equal(pg.astype(np.int64).sum(-1), pc)
    st = np.float32(rng.uniform(0.01, 1, M))
    sw = np.float32(rng.uniform(1e-4, 1e-3, N))
    pg = orc.gemm_acc(xq, w, 8, 64)
    y_pg = orc.dequant(pg, st, np.repeat(sw[:, None], K // 64, 1))
    y_pc = orc.dequant(pc, st, sw)
    assert np.array_equal(y_pg.view(np.uint16), y_pc.view(np.uint16))


# --------------------------------------------------------------- dequant ---

def _ordered(h):
    """fp16 values as integers in value order, one step per ulp; +0 and -0 coincide."""
    b = np.asarray(h, np.float16).view(np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _unpack4(wq4):
    q = np.empty((wq4.shape[0], wq4.shape[1] * 2), np.int64)
    q[:, 0::2] = (wq4 & 0xF).astype(np.int64) - 8
    q[:, 1::2] = (wq4 >> 4).astype(np.int64) - 8
    return q


def pin_dequant_vs_fake_quant(orc):
    """Whole path equals the dequantize-then-multiply form: fp16 of
    (xq * s_tok) @ (wq * s_w)^T evaluated by numpy in float64; per channel, per
    group and int4.  The two differ only by float64 rounding, so at most one
    fp16 ulp apart on near-ties and identical almost everywhere."""
    from synth_inputs import activations, weights
    M, N, K = 16, 48, 512
    x = activations(M, K, seed=11)
    w = weights(N, K, seed=11)
    for bits, gs in ((8, 0), (8, 64), (8, 128), (4, 0), (4, 64), (4, 128)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        y, xq, st = orc.linear(x, wq, sw, bits, gs)
        codes = wq.astype(np.int64) if bits == 8 else _unpack4(wq)
        L = K if gs == 0 else gs
        sw_full = np.repeat(np.asarray(sw, np.float64).reshape(N, -1), L, axis=1)
        xd = xq.astype(np.float64) * st.astype(np.float64)[:, None]
        wd = codes.astype(np.float64) * sw_full
        ref = (xd @ wd.T).astype(np.float16)
        yb, rb = _ordered(y), _ordered(ref)
        assert np.max(np.abs(yb - rb)) <= 1, (bits, gs)
        assert np.mean(yb == rb) > 0.999, (bits, gs)
        # quantize_act alone agrees with the whole path's quantization
        xq2, st2 = orc.quantize_act(x)
        assert np.array_equal(xq2, xq) and np.array_equal(st2, st)


def _nearest_16(bits16, exact, dtype):
    """True when the 16-bit pattern (fp16 dtype 0, bf16 dtype 1) is a value
    nearest to the exact rational: no neighbouring pattern is closer."""
    from fractions import Fraction
    def val(b):
        b = int(b) & 0xFFFF
        if dtype == 0:
            return Fraction(float(np.array([b], np.uint16).view(np.float16)[0]))
        return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))
    got = val(bits16)
    mag = int(bits16) & 0x7FFF
    sign = int(bits16) & 0x8000
    near = [sign | (mag + 1)]
    near.append(sign | (mag - 1) if mag else (sign ^ 0x8000) | 1)
    return all(abs(got - exact) <= abs(val(b) - exact) for b in near)


def pin_dequant_nearest_rational(orc):
    """The dequant, from the oracle's own codes and scales: every fp16 and
    bf16 output is a value nearest to the exact rational
    s_tok[m] * sum_g s_w[n, g] * acc[m, n, g] (Python fractions; fp32 scales
    are exact rationals), per channel, per group 64 / 128 and int4.  A dropped
    scale, a wrong group index or a transposed scale fails it."""
    from fractions import Fraction
    from synth_inputs import activations, weights
    M, N, K = 5, 7, 256
    x = activations(M, K, seed=47)
    w = weights(N, K, seed=47)
    xq, st = orc.quantize_act(x)
    for bits, gs in ((8, 0), (8, 64), (8, 128), (4, 0), (4, 64)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        acc = orc.gemm_acc(xq, wq, bits, gs)
        a3 = acc if acc.ndim == 3 else acc[:, :, None]
        swf = np.asarray(sw, np.float32).reshape(N, -1)
        outs = [orc.dequant_ex(acc, st, sw, d) for d in (0, 1)]
        for m in range(M):
            for n in range(N):
                exact = Fraction(float(st[m])) * sum(Fraction(float(swf[n, g])) * int(a3[m, n, g])
                                                     for g in range(a3.shape[2]))
                for d in (0, 1):
                    assert _nearest_16(outs[d][m, n], exact, d), (bits, gs, m, n, d)


def pin_symmetry(orc):
    """quantize(-X) = -quantize(X) and Y(-X) = -Y(X), bit for bit."""
    from synth_inputs import activations, weights
    x = activations(8, 256, seed=3)
    w = weights(32, 256, seed=3)
    for bits, gs in ((8, 0), (8, 64), (4, 0), (4, 64)):
        wq, sw = orc.quantize_weight(w, bits, gs)
        y, xq, st = orc.linear(x, wq, sw, bits, gs)
        yn, xqn, stn = orc.linear(-x, wq, sw, bits, gs)
        assert np.array_equal(xqn, -xq) and np.array_equal(stn, st)
        assert np.array_equal(yn.view(np.uint16), (-y).view(np.uint16))
    wq, sw = orc.quantize_weight(w, 8, 0)
    wqn, swn = orc.quantize_weight(-w, 8, 0)
    assert np.array_equal(wqn, -wq) and np.array_equal(swn, sw)


def pin_power_of_two_scaling(orc):
    """X * 2^j (no fp16 over/underflow) leaves the codes unchanged and scales
    s_tok and Y by exactly 2^j."""
    from synth_inputs import activations, weights
    x = activations(6, 256, seed=4)
    w = weights(40, 256, seed=4)
    wq, sw = orc.quantize_weight(w, 8, 0)
    y, xq, st = orc.linear(x, wq, sw)
    for j in (-3, 2):
        xs = (x.astype(np.float32) * np.float32(2.0 ** j)).astype(np.float16)
        ys, xqs, sts = orc.linear(xs, wq, sw)
        assert np.array_equal(xqs, xq)
        assert np.array_equal(sts, st * np.float32(2.0 ** j))
        big = np.abs(y.astype(np.float32)) > 2.0 ** -10
        assert np.array_equal(ys.astype(np.float64)[big], y.astype(np.float64)[big] * 2.0 ** j)


def pin_identity_weight(orc):
    """W = c * I with c = 127/128: each row's only nonzero is c, so s_w = 1/128
    and the code is 127; then y[m, n] = xq[m, n] * s_tok[m] * 127/128."""
    from synth_inputs import activations
    K = 128
    x = activations(4, K, seed=5)
    c = 127.0 / 128.0
    w = _f16(np.eye(K) * c)
    wq, sw = orc.quantize_weight(w, 8, 0)
    assert np.all(sw == np.float32(1 / 128.0)) and np.array_equal(np.diag(wq), np.full(K, 127))
    y, xq, st = orc.linear(x, wq, sw)
    ref = (xq.astype(np.float64) * st.astype(np.float64)[:, None] * c).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def pin_quality_vs_fp16_gemm(orc):
    """On the small per-channel workload (M=64, N=512, K=1024, seed 0) the
    quantized output tracks the unquantized product: cosine about 0.9991 (the
    outlier columns inflate the per-token scale), relative error a few percent."""
    from synth_inputs import activations, weights
    x = activations(64, 1024)
    w = weights(512, 1024)
    wq, sw = orc.quantize_weight(w, 8, 0)
    y, _, _ = orc.linear(x, wq, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    yv = y.astype(np.float64)
    cos = float((yv * ref).sum() / np.sqrt((yv * yv).sum() * (ref * ref).sum()))
    rel = float(np.linalg.norm(yv - ref) / np.linalg.norm(ref))
    assert 0.9985 < cos < 0.99975, cos
    assert rel < 0.06, rel


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
