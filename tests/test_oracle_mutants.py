"""Plant plausible mistakes into copies of the oracle's source; the pins must catch each one.

A mutant is the oracle's C source with one textual substitution, compiled with
gcc into a temporary directory.  Nothing here runs on a GPU.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pin_suite as suite

SRC = os.path.join(os.path.dirname(oracle.__file__), "q4_oracle.c")

MUTANTS = {
    "offset_7_not_8": ("(double)(code - 8)", "(double)(code - 7)"),
    "sign_flipped": ("(double)(code - 8)", "(double)(8 - code)"),
    "nibbles_swapped": ("(k < 16) ? (byte & 0x0F) : (byte >> 4)", "(k < 16) ? (byte >> 4) : (byte & 0x0F)"),
    "sequential_nibbles": ("blk[2 + (k & 15)]", "blk[2 + (k >> 1)]"),
    "scale_big_endian": ("blk[0] | ((uint16_t)blk[1] << 8)", "blk[1] | ((uint16_t)blk[0] << 8)"),
    "magnitude_without_abs": ("mag[mm] += fabs(p);", "mag[mm] += p;"),
    "f16_bias_off_by_one": ("e - 25", "e - 24"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "block_stride_16": ("(i / 32) * 18", "(i / 32) * 16"),
    "output_transposed": ("y[mm * nrows + n] = acc[mm];", "y[n * m + mm] = acc[mm];"),
    "argmax_last_tie": ("if (y[i] > y[best])", "if (y[i] >= y[best])"),
    "scale_dropped": ("return (double)(code - 8) * d;", "return (double)(code - 8);"),
    "x_ignored_sign": ("xt[i * m + mm] = q4o_f16_to_f64(xr[i]);", "xt[i * m + mm] = fabs(q4o_f16_to_f64(xr[i]));"),
    "activation_row_stride": ("xt[i * m + mm] = q4o_f16_to_f64(xr[i]);", "xt[i * m + mm] = q4o_f16_to_f64(xr[i ^ 1]);"),
    "weight_column_shifted": ("const double* xi = xt + i * m;", "const double* xi = xt + ((i + 1) % k) * m;"),
    "prefix_counts_all_matches": ("while (i < m && tokens[i] == draft[i]) ++i;",
                                  "for (int64_t j = 0; j < m; ++j) i += tokens[j] == draft[j];"),
    "norm_sum_not_mean": ("sqrt(ss / (double)k + eps)", "sqrt(ss + eps)"),
    "norm_eps_outside_root": ("1.0 / sqrt(ss / (double)k + eps)", "1.0 / (sqrt(ss / (double)k) + eps)"),
    "norm_root_missing": ("1.0 / sqrt(ss / (double)k + eps)", "1.0 / (ss / (double)k + eps)"),
    "norm_gain_ignored": ("q4o_f16_to_f64(h[i]) * q4o_f16_to_f64(g[i]) * r", "q4o_f16_to_f64(h[i]) * r"),
    "norm_gain_reversed": ("q4o_f16_to_f64(g[i]) * r", "q4o_f16_to_f64(g[k - 1 - i]) * r"),
    "norm_sum_of_abs": ("ss += hi * hi;", "ss += fabs(hi);"),
    "f16_ties_away_from_zero": ("(rem == 0.5 && fmod(q, 2.0) != 0.0)", "(rem == 0.5)"),
    "f16_truncates": ("if (rem > 0.5 || (rem == 0.5 && fmod(q, 2.0) != 0.0)) q += 1.0;", ""),
    "f16_overflow_saturates": ("if (a >= 65520.0) return sign | 0x7C00;", "if (a >= 65520.0) return sign | 0x7BFF;"),
    "f16_overflow_threshold_65504": ("if (a >= 65520.0)", "if (a > 65504.0)"),
    "f16_subnormal_quantum": ("if (E < -14) E = -14;", "if (E < -15) E = -15;"),
    "f16_carry_lost": ("q = 1024.0;\n        E += 1;", "q = 2047.0;"),
    "f16_sign_dropped": ("const uint16_t sign = signbit(v) ? 0x8000 : 0;", "const uint16_t sign = 0;"),
    "handoff_residual_dropped": ("q4o_f64_to_f16((r ? (double)r[n] : 0.0) + y[n])", "q4o_f64_to_f16(y[n])"),
    "handoff_residual_subtracted": ("q4o_f64_to_f16((r ? (double)r[n] : 0.0) + y[n])",
                                    "q4o_f64_to_f16(y[n] - (r ? (double)r[n] : 0.0))"),
    "handoff_rounded_before_residual": ("q4o_f64_to_f16((r ? (double)r[n] : 0.0) + y[n])",
                                        "q4o_f64_to_f16((r ? (double)r[n] : 0.0) + q4o_f16_to_f64(q4o_f64_to_f16(y[n])))"),
    "q8_codes_unsigned": ("const int code = (int)(int8_t)blk[2 + kk];", "const int code = (int)blk[2 + kk];"),
    "q8_codes_offset_128": ("const int code = (int)(int8_t)blk[2 + kk];", "const int code = (int)blk[2 + kk] - 128;"),
    "q8_scale_big_endian": ("q4o_f16_to_f64((uint16_t)(blk[0] | ((uint16_t)blk[1] << 8)));\n    const int code",
                            "q4o_f16_to_f64((uint16_t)(blk[1] | ((uint16_t)blk[0] << 8)));\n    const int code"),
    "q8_block_stride_32": ("row + (i / 32) * 34, (int)(i % 32)", "row + (i / 32) * 32, (int)(i % 32)"),
    "q8_codes_shifted": ("const int code = (int)(int8_t)blk[2 + kk];", "const int code = (int)(int8_t)blk[1 + kk];"),
    "prefix_past_mismatch": ("while (i < m && tokens[i] == draft[i]) ++i;",
                             "while (i < m && tokens[i] == draft[i]) ++i;\n    if (i < m) ++i;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, "mutation site vanished from the oracle: " + old
    mutated = src.replace(old, new)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so), str(c), "-lm"])
    bad = suite.failures(oracle.Oracle(str(so)))
    assert bad, "mutant %s passed every pin" % name


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "libcopy.so"
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so), SRC, "-lm"])
    assert suite.failures(oracle.Oracle(str(so))) == []
