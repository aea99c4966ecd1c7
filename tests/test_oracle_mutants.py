"""The pins are strong enough: each planted mistake in a copy of the oracle
fails at least one of them (no GPU).

Every mutant is a one-line edit of q4_oracle.c made in a temporary directory
and compiled with the oracle's own flags; the oracle under oracle/ is never
touched.
"""
import os

import pytest

import oracle
import oracle_pins

# (name, original text, planted mistake)
MUTANTS = [
    ("divisor_8", "amax / 7.0f", "amax / 8.0f"),
    ("nibble_order_pack", "(uint8_t)((q_even + 8) | ((q_odd + 8) << 4))",
     "(uint8_t)((q_odd + 8) | ((q_even + 8) << 4))"),
    ("round_truncate", "nearbyintf(w / s)", "truncf(w / s)"),
    ("round_half_away", "nearbyintf(w / s)", "roundf(w / s)"),
    ("clamp_symmetric", "return -8;\n    if", "return -7;\n    if"),
    ("no_zero_scale_rule", "if (s == 0.0f)\n        return 0;", ""),
    ("signed_max", "float a = fabsf(g[t]);", "float a = g[t];"),
    ("f16_round_half_up",
     "if (rem > 0x1000u || (rem == 0x1000u && (r & 1u)))",
     "if (rem >= 0x1000u)"),
    ("f16_subnormal_cut", "if (shift > 24)", "if (shift > 23)"),
    ("f16_widen_bias", "ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    ("divide_by_unrounded_scale", "float s = (float)q4o_f16_to_f64(s16);", "float s = ratio;"),
    ("product_drops_scale", "acc += s * dot;", "acc += dot;"),
    ("product_nibble_order", "(kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
     "(kk % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    ("product_table_offset", "(double)kLevel[code]", "(double)(code - 7)"),
    ("product_scale_index", "scales[r * G + j]);\n                double dot",
     "scales[r * G + (j + 1) % G]);\n                double dot"),
    ("product_x_transposed", "const double* xi = xd + i * k;", "const double* xi = xd + i;"),
    ("product_sign", "double term = xi[kk] *", "double term = -xi[kk] *"),
    ("product_dropped_term", "for (int t = 0; t < 32; ++t) {\n                    int64_t kk",
     "for (int t = 0; t < 31; ++t) {\n                    int64_t kk"),
    ("bound_not_absolute", "acc_abs += fabs(s) * dot_abs;", "acc_abs += fabs(s * dot);"),
    ("output_index", "y[i * n + r] = acc;", "y[r * m + i] = acc;"),
    ("f16_sign", "double prod = xrow[t] *", "double prod = -xrow[t] *"),
    ("f16_weight_index", "const uint16_t* row = w + r * k;", "const uint16_t* row = w + r;"),
    ("f16_dropped_term", "for (int64_t t = 0; t < k; ++t) {\n                double prod",
     "for (int64_t t = 1; t < k; ++t) {\n                double prod"),
    ("f16_bound_not_absolute", "sum_abs += fabs(prod);", "sum_abs += prod;"),
    ("f16_output_index", "y[i * n + r] = sum;", "y[r * m + i] = sum;"),
    ("f16_widened_as_zero_exponent", "double prod = xrow[t] * q4o_f16_to_f64(row[t]);",
     "double prod = xrow[t] * (double)row[t];"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as fh:
        return fh.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, "mutation anchor not unique: %s" % name
    src = tmp_path / ("q4_oracle_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib = oracle.compile_oracle(str(src), str(tmp_path / ("lib_%s.so" % name)))
    # the mutant needs the oracle header next to it
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
