"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c, makes one plausible mistake (a dropped term, a wrong
sign or index, eps outside the root, a wrong rounding rule, the FNUZ fp8
maximum instead of the OCP one), builds the copy with the same flags and runs
every pin against it. At least one pin has to fail; otherwise the pins would
not notice that mistake in the real oracle either. Every mutation keeps memory
accesses in bounds.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_residual": ("x[h] = rv + s[h];", "x[h] = s[h];"),
    "residual_sign": ("x[h] = rv + s[h];", "x[h] = s[h] - rv;"),
    "partial_sign": ("      s[h] += c;\n      mag[h] += fabs(c);\n    }\n  }\n}\n\n/*\n * Complete owed work, deferred",
                     "      s[h] -= c;\n      mag[h] += fabs(c);\n    }\n  }\n}\n\n/*\n * Complete owed work, deferred"),
    "drop_first_partial": ("for (int p = 0; p < P; ++p)", "for (int p = 1; p < P; ++p)"),
    "partial_row_index": ("partials[p] + t * ld", "partials[p] + (t == 0 ? 0 : t - 1) * ld"),
    "reversed_hidden_index": ("double c = orc_bf16_value(row[h]);", "double c = orc_bf16_value(row[H - 1 - h]);"),
    "gate_ignored": ("double c = g * orc_bf16_value(row[h]);", "double c = orc_bf16_value(row[h]);"),
    "gate_pairing": ("double g = (double)gate[t * k + j];", "double g = (double)gate[t * k + (k - 1 - j)];"),
    "eps_outside_root": ("return 1.0 / sqrt(sum_sq / (double)H + (double)eps);",
                         "return 1.0 / (sqrt(sum_sq / (double)H) + (double)eps);"),
    "eps_dropped": ("return 1.0 / sqrt(sum_sq / (double)H + (double)eps);",
                    "return 1.0 / sqrt(sum_sq / (double)H);"),
    "sum_not_mean": ("return 1.0 / sqrt(sum_sq / (double)H + (double)eps);",
                     "return 1.0 / sqrt(sum_sq + (double)eps);"),
    "weight_dropped": ("y[h] = x[h] * inv * scale;", "y[h] = x[h] * inv;"),
    "norm_of_rounded_snapshot": ("y[h] = x[h] * inv * scale;",
                                 "y[h] = orc_bf16_value(orc_bf16_round(x[h])) * inv * scale;"),
    "gemma_offset_ignored": ("double scale = gemma ? 1.0 + (double)w[h] : (double)w[h];",
                             "double scale = (double)w[h];"),
    "gemma_everywhere": ("double scale = gemma ? 1.0 + (double)w[h] : (double)w[h];",
                         "double scale = 1.0 + (double)w[h];"),
    "bf16_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(n_r, 2.0) != 0.0)) n_r += 1.0;\n    r = n_r * step;\n  }\n  float f",
                       "if (frac >= 0.5) n_r += 1.0;\n    r = n_r * step;\n  }\n  float f"),
    "bf16_truncate": ("if (frac > 0.5 || (frac == 0.5 && fmod(n_r, 2.0) != 0.0)) n_r += 1.0;\n    r = n_r * step;\n  }\n  float f",
                      "r = n_r * step;\n  }\n  float f"),
    "e4m3_subnormal_step": ("if (e < -6) e = -6;", "if (e < -7) e = -7;"),
    "e4m3_bias": ("v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    "fnuz_max": ("const float scale = amax / 448.0f;", "const float scale = amax / 240.0f;"),
    "scale_inverted": ("float v = (float)y[h] / scale;", "float v = (float)y[h] * scale;"),
    "fp8_decided_in_fp64": ("float v = (float)y[h] / scale;\n    if (v > 448.0f) v = 448.0f;\n"
                            "    if (v < -448.0f) v = -448.0f;",
                            "double v = y[h] / (double)scale;\n    if (v > 448.0) v = 448.0;\n"
                            "    if (v < -448.0) v = -448.0;"),
    "moe_index_ignored": ("int64_t e = idx[t * k + j];", "int64_t e = t * k + j;"),
    "invalid_pick_clamped": ("if (e < 0 || e >= n_rows) continue;", "if (e < 0 || e >= n_rows) e = 0;"),
    "partials_slice_relative": ("complete_partials_row(H, P, partials, ld_p, row_begin + i, b.s, b.mag);\n    apply_update_row",
                                "complete_partials_row(H, P, partials, ld_p, i, b.s, b.mag);\n    apply_update_row"),
    "moe_slice_relative": ("complete_moe_row(H, k, E, ld_e, n_rows_e, idx, gate, row_begin + i, b.s, b.mag);\n    apply_update_row",
                           "complete_moe_row(H, k, E, ld_e, n_rows_e, idx, gate, i, b.s, b.mag);\n    apply_update_row"),
    "extra_dropped": ("if (extra) add_extra_row(H, extra + (row_begin + i) * ld_x, b.s, b.mag);",
                      "(void)extra;"),
    "extra_not_global_row": ("if (extra) add_extra_row(H, extra + (row_begin + i) * ld_x, b.s, b.mag);",
                             "if (extra) add_extra_row(H, extra + i * ld_x, b.s, b.mag);"),
    "snapshot_drops_residual": ("apply_update_row(H, residual ? residual + i * ld_r : NULL, b.s, b.x, b.mag);\n    store_bf16_row(H, b.x, out + i * ld_o);",
                                "apply_update_row(H, NULL, b.s, b.x, b.mag);\n    store_bf16_row(H, b.x, out + i * ld_o);"),
}


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, name, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} not found in oracle.c"
    mutated = source.replace(old, new, 1)
    src = tmp_path / "oracle_mutant.c"
    src.write_text(mutated)
    lib_path = str(tmp_path / "liboracle_mutant.so")
    oracle.build(str(src), lib_path)
    o = oracle.Oracle(oracle.load(lib_path))
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
