"""The quantizer's fast rule, replayed in numpy float32 on the CPU.

The quantize kernels compute each code as rint(fl32(x * rs)) with
rs = fl32(1 / s) and fall back to the correctly rounded quotient fl32(x / s)
for a chunk of 8 values when any product lies within 2^-14 of a
half-integer, or when s is not a normal fp32 number (s < 2^-126).  These
tests replay that rule with IEEE float32 numpy arithmetic (subnormals kept)
and hold it against the oracle's codes, which always divide:

* with the tiny-scale fallback the rule agrees with the oracle on rows of
  every magnitude, down to the smallest bf16 value;
* without it, rows whose scale is below 2^-128 (reciprocal +inf) get wrong
  codes: the fallback is needed (between 2^-128 and 2^-126 it is only
  conservative);
* for normal scales the product's distance to the quotient stays below the
  2^-15.4 bound the near-half test relies on.
"""
import numpy as np

from oracle.oracle import get as get_oracle
from tests.gpu_util import bf16_bits

F32 = np.float32


def _rule_codes(x32: np.ndarray, s: np.float32, tiny_fallback: bool = True) -> np.ndarray:
    """Codes of one row of float32 values by the kernel's rule."""
    with np.errstate(all="ignore"):
        rs = F32(1.0) / s
        t = (x32 * rs).astype(F32)
        d = t - np.rint(t)
        near = np.abs(np.abs(d) - F32(0.5)) < F32(2.0 ** -14)
        chunk_near = near.reshape(-1, 8).any(axis=1)
        if tiny_fallback and not (s >= F32(2.0 ** -126)):
            chunk_near[:] = True
        q = (x32 / s).astype(F32)
        t = np.where(np.repeat(chunk_near, 8), q, t)
        r = np.rint(t)
        r = np.where(np.isnan(r), F32(-127), r)          # maxNum/minNum send NaN to a bound
        r = np.clip(r, -127, 127)
    return np.zeros_like(r, dtype=np.int8) if s == 0 else r.astype(np.int8)


def _rows(amaxes, K, seed):
    rng = np.random.default_rng([seed, 5])
    out = []
    for a in amaxes:
        r = rng.standard_normal(K)
        r = r / np.abs(r).max() * a
        r[:8] = [0.0, a, -a, a / 2, -a / 2, a / 4, 0.0, -a]
        out.append(r.astype(F32))
    return np.stack(out)


AMAX = [1e-36, 3e-37, 1e-37, 1e-38, 2.0 ** -133, 1e-30, 1.0, 3.7, 100.0, 1e20] + list(
    10.0 ** np.random.default_rng(3).uniform(-38, 30, 40))


def test_rule_matches_oracle_at_every_magnitude():
    orc = get_oracle()
    K = 256
    xb = bf16_bits(_rows(AMAX, K, 1))
    rq, rs = orc.quantize_act_ex(xb, 1, K=K)
    x32 = (xb.astype(np.uint32) << 16).view(F32)
    tiny = 0
    for i in range(xb.shape[0]):
        s = rs[i]
        assert s == F32(np.abs(x32[i]).max()) / F32(127.0)
        tiny += bool(0 < s < 2.0 ** -126)
        assert np.array_equal(_rule_codes(x32[i], s), rq[i]), "row %d (scale %g)" % (i, s)
    assert tiny >= 4


def test_rule_without_tiny_fallback_fails_below_normal_scales():
    """The fallback is not decorative: drop it and the codes of rows with
    scales below 2^-128 collapse to +-127 (zeros to -127)."""
    orc = get_oracle()
    K = 256
    xb = bf16_bits(_rows([3e-37, 1e-37, 2.0 ** -133], K, 2))
    rq, rs = orc.quantize_act_ex(xb, 1, K=K)
    x32 = (xb.astype(np.uint32) << 16).view(F32)
    for i in range(xb.shape[0]):
        assert rs[i] < 2.0 ** -128
        bad = _rule_codes(x32[i], rs[i], tiny_fallback=False)
        assert not np.array_equal(bad, rq[i])
        assert bad[0] == -127 and rq[i][0] == 0          # a zero value
    # scales between 2^-128 and 2^-126 have finite reciprocals: the product
    # rule would still hold there, so the fallback's threshold at the
    # smallest normal number is conservative (it costs only such rare rows)
    rng = np.random.default_rng(8)
    amax = rng.uniform(127 * 2.0 ** -127.9, 127 * 2.0 ** -126, 64)
    xb = bf16_bits(_rows(amax, K, 4))
    rq, rs = orc.quantize_act_ex(xb, 1, K=K)
    x32 = (xb.astype(np.uint32) << 16).view(F32)
    assert np.all((rs > 2.0 ** -128) & (rs < 2.0 ** -126))
    for i in range(len(rs)):
        assert np.array_equal(_rule_codes(x32[i], rs[i], tiny_fallback=False), rq[i])
        assert np.array_equal(_rule_codes(x32[i], rs[i]), rq[i])


def test_product_error_bound_for_normal_scales():
    """|fl32(x * fl32(1/s)) - fl32(x / s)| < 2^-15.4 whenever s is a normal
    fp32 number and |x / s| <= 127.5 (the absmax row's own quotients)."""
    rng = np.random.default_rng(9)
    worst = 0.0
    for e in rng.uniform(-118.9, 120, 300):
        a = F32(2.0 ** e)
        x = (rng.uniform(-1, 1, 4096) * a).astype(F32)
        s = F32(np.abs(x).max()) / F32(127.0)
        assert s >= 2.0 ** -126
        prod = (x * (F32(1.0) / s)).astype(F32).astype(np.float64)
        quot = (x / s).astype(F32).astype(np.float64)
        worst = max(worst, float(np.abs(prod - quot).max()))
    assert worst < 2.0 ** -15.4, worst
