"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutation below is a plausible slip in a quantized-linear reference (a
wrong divisor, a rounding mode, a swapped nibble, a transposed index, a dropped
scale ...).  Each is applied textually to a temporary copy of
``oracle/cider_oracle.c``, compiled with gcc, and the full pin set of
``tests/oracle_pins.py`` is run against it; the test passes only if some pin
rejects the mutant.  All of this runs on the CPU.
"""
import os

import pytest

from oracle.oracle import SOURCE, Oracle, compile_oracle
from tests import oracle_pins

MUTATIONS = {
    "scale_divisor_128": ("float s = range / qmax;", "float s = range / (qmax + 1.0f);"),
    "round_half_away": ("float r = nearbyintf(t);", "float r = roundf(t);"),
    "reciprocal_multiply": ("/ s;  /* fp32 quotient */", "* (1.0f / s);"),
    "truncate_not_round": ("float r = nearbyintf(t);", "float r = truncf(t);"),
    "signed_absmax": ("float a = fabsf(v[i]);", "float a = v[i];"),
    "nibble_order_pack": ("(uint8_t)(u_even | (u_odd << 4))", "(uint8_t)(u_odd | (u_even << 4))"),
    "nibble_order_unpack": ("(k % 2 == 0) ? (b & 0xf) : (b >> 4)", "(k % 2 == 1) ? (b & 0xf) : (b >> 4)"),
    "zero_point_7": ("return u - 8;", "return u - 7;"),
    "pack_no_zero_point": ("int u_even = qbuf[2 * j] + 8;", "int u_even = qbuf[2 * j] + 0;"),
    "int4_divisor_8": ("float qmax = bits == 8 ? 127.0f : 7.0f;", "float qmax = bits == 8 ? 127.0f : 8.0f;"),
    "weight_row_index": ("s += (int64_t)xrow[k] * weight_code(wq, bits, K, n, k);",
                         "s += (int64_t)xrow[k] * weight_code(wq, bits, K, n ? n - 1 : 0, k);"),
    "group_offset_dropped": ("const uint16_t *run = w + n * K + g * gs;", "const uint16_t *run = w + n * K;"),
    "group_range_off_by_one": ("g * gs, (g + 1) * gs);", "g * gs, (g + 1) * gs - 1);"),
    "group_scale_transposed": ("t += (double)s_w_row[g] * (double)acc_row[g];",
                               "t += (double)s_w_row[0] * (double)acc_row[g];"),
    "token_scale_dropped": ("return (double)s_tok * t;", "return t;"),
    "group_sum_shifted": ("t += (double)s_w_row[g] * (double)acc_row[g];",
                          "t += (double)s_w_row[g] * (double)acc_row[g ? g - 1 : 0];"),
    "token_scale_squared": ("return (double)s_tok * t;", "return (double)s_tok * (double)s_tok * t * 64.0;"),
    "half_decode_exponent": ("ldexp((double)(1024 + man), e - 25)", "ldexp((double)(1024 + man), e - 24)"),
    "half_encode_ties_away": ("double m = nearbyint(ldexp(a, -q));", "double m = round(ldexp(a, -q));"),
    "half_encode_quantum": ("? -24 : e - 11;", "? -24 : e - 10;"),
    "half_encode_subnormal_quantum": ("? -24 : e - 11;", "? -23 : e - 11;"),
    "scale_in_fp16": ("float s = range / qmax;", "float s = (float)oracle_half_to_double(oracle_double_to_half(range / qmax));"),
    "percentile_rank_n": ("double h = (double)(n - 1) * (p / 100.0);", "double h = (double)n * (p / 100.0);"),
    "percentile_lower_value": ("return g >= 0.5 ? b - d * (1.0 - g) : a + d * g;", "return a;"),
    "percentile_one_formula": ("return g >= 0.5 ? b - d * (1.0 - g) : a + d * g;", "return a + d * g;"),
    "percentile_signed": ("buf[i] = fabs((double)v[i]);", "buf[i] = (double)v[i];"),
    "clip_range_not_rounded": ("float range = clip ? (float)percentile_abs(v, gs, clip_percentile, buf)",
                               "float range = clip ? (float)(percentile_abs(v, gs, clip_percentile, buf) * (1.0 + 1e-7))"),
    "smooth_multiplies": ("v[i] = smooth ? f / smooth[i] : f;", "v[i] = smooth ? f * smooth[i] : f;"),
    "smooth_ignored": ("v[i] = smooth ? f / smooth[i] : f;", "v[i] = f;"),
    "smooth_channel_shifted": ("v[i] = smooth ? f / smooth[i] : f;", "v[i] = smooth ? f / smooth[i ? i - 1 : 0] : f;"),
    "fold_divides": ("* (double)smooth[k], dtype);", "/ (double)smooth[k], dtype);"),
    "fold_via_fp32": ("narrow((double)widen(w[n * K + k], dtype) * (double)smooth[k], dtype);",
                      "narrow((double)(widen(w[n * K + k], dtype) * smooth[k]), dtype);"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "bf16_encode_quantum": ("-133 : e - 8;", "-133 : e - 7;"),
    "bf16_encode_ties_away": ("double m = nearbyint(ldexp(a, -q));           /* count of quanta, ties to even */\n    if (q == -133)",
                              "double m = round(ldexp(a, -q));\n    if (q == -133)"),
    "bf16_encode_bias": ("((q + 134) << 7)", "((q + 133) << 7)"),
    "decode_group_scale_index": ("t += (double)s_w[n * G + g] * a;", "t += (double)s_w[n * G] * a;"),
    "decode_quantizes_nothing_wrong_sign": ("a += (double)widen(x[k], x_dtype) * (double)weight_code(wq, bits, K, n, k);",
                                           "a += (double)widen(x[k], x_dtype) * (double)abs(weight_code(wq, bits, K, n, k));"),
    "decode_x_dtype_ignored": ("a += (double)widen(x[k], x_dtype)", "a += (double)widen(x[k], DT_F16)"),
    "output_dtype_ignored": ("narrow(dequant_value(s_tok[m], s_w + n * G, acc + (m * N + n) * G, G),\n                                  y_dtype);",
                             "narrow(dequant_value(s_tok[m], s_w + n * G, acc + (m * N + n) * G, G),\n                                  DT_F16);"),
    "dequant_via_float": ("return (double)s_tok * t;",
                          "return (double)(float)((float)s_tok * (float)t) * 1.0001;"),
}


def _mutant(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SOURCE).read()
    assert src.count(old) >= 1, "mutation %s no longer matches the oracle source" % name
    mutated = src.replace(old, new)
    path = os.path.join(str(tmp_path), "mut_%s.c" % name)
    with open(path, "w") as f:
        f.write(mutated)
    return Oracle(compile_oracle(path, path[:-2] + ".so"))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, name):
    orc = _mutant(tmp_path, name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # AssertionError or an oracle error code
            caught.append("%s: %s" % (pin.__name__, type(e).__name__))
    assert caught, "no pin caught the planted mistake %r" % name
