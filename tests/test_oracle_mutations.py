"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (on the CPU only),
compiles the mutant, swaps it in for the real library and reruns a set of the
pins from test_oracle_pins.  Every mutant must fail at least one of them.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_pins_ext as pins_ext

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "nbw_oracle.c")

MUTANTS = {
    "lsb_first_planes": ("(codes[i * k + j] >> (7 - p)) & 1", "(codes[i * k + j] >> p) & 1"),
    "natural_bit_order": ("(int)(e / 2 + 16 * (e % 2))", "(int)e"),
    "group_major_tiles": ("((i / 16) * groups + g) * 256",
                          "(g * (padded_rows(n) / 16) + i / 16) * 256"),
    "dropped_half": ("((double)q + 0.5 - ldexp(1.0, r - 1))", "((double)q - ldexp(1.0, r - 1))"),
    "wrong_exponent": ("s * ldexp(1.0, 8 - r)", "s * ldexp(1.0, 7 - r)"),
    "shifted_scale_group": ("double s = nbwo_bf16_to_double(scales[i * groups + j / 128]);\n        wrow",
                            "double s = nbwo_bf16_to_double(scales[i * groups + (j / 128 + 1) % groups]);\n        wrow"),
    "transposed_x": ("acc += nbwo_bf16_to_double(x[b * k + j]) * wrow[j];",
                     "acc += nbwo_bf16_to_double(x[j * batch + b]) * wrow[j];"),
    "asym_transposed_x": ("acc += wrow[j] * nbwo_bf16_to_double(x[b * k + j]);",
                          "acc += wrow[j] * nbwo_bf16_to_double(x[j * batch + b]);"),
    "wrong_sign": ("acc += nbwo_bf16_to_double", "acc -= nbwo_bf16_to_double"),
    "lsb_first_unpack": ("v = 2 * v + read_bit(planes, n, k, p, i, j);",
                         "v = v + (read_bit(planes, n, k, p, i, j) << p);"),
    "padding_rows_ones": ("for (int64_t i = 0; i < n; ++i)\n            for (int64_t j = 0; j < k; ++j) {\n"
                          "                int b = (codes[i * k + j] >> (7 - p)) & 1;",
                          "for (int64_t i = 0; i < padded_rows(n); ++i)\n            for (int64_t j = 0; j < k; ++j) {\n"
                          "                int b = i < n ? ((codes[i * k + j] >> (7 - p)) & 1) : 1;"),
    "sampled_row_shifted": ("qgemm_row(x, batch, planes, scales, n, k, r, rows[t], wrow, y + t, nrows);",
                            "qgemm_row(x, batch, planes, scales, n, k, r, (rows[t] + 1) % n, wrow, y + t, nrows);"),
    # asymmetric children
    "asym_dropped_half": ("((double)q + 0.5) - 0.5 - z)", "((double)q + 0.5) - z)"),
    "asym_zero_sign": ("((double)q + 0.5) - 0.5 - z)", "((double)q + 0.5) - 0.5 + z)"),
    "asym_zero_of_next_group": ("zeros[i * groups + j / 128]",
                                "zeros[i * groups + (j / 128 + 1) % groups]"),
    # code chooser
    "choose_last_of_ties": ("if (c == 0 || loss < best_loss)", "if (c == 0 || loss <= best_loss)"),
    "choose_wrong_child_shift": ("nbwo_dequant_value(s, c >> (8 - r), r)",
                                 "nbwo_dequant_value(s, c >> (7 - r), r)"),
    "choose_ignores_lambda": ("double term = lambdas[t] * e2;", "double term = e2;"),
}


def _pin_calls():
    calls = [pins.test_pack_roundtrip_r8_reconstructs_parent,
             lambda: pins.test_child_codes_are_msb_slices(3),
             lambda: pins.test_child_value_is_mean_of_parent_bucket(2),
             pins.test_dequant_r8_is_parent_grid,
             lambda: pins.test_qgemm_exact_rational_bruteforce(3),
             lambda: pins.test_qgemm_second_route_without_planes(4),
             lambda: pins.test_qgemm_identity_activations_give_weights(4),
             pins.test_padding_rows_are_zero_bits,
             pins.test_qgemm_rows_equals_full]
    for row in pins._golden_layout():
        calls.append(lambda row=row: pins.test_layout_worked_examples(*row))
    calls += [lambda: pins_ext.test_asym_with_midpoint_zero_is_symmetric(3),
              pins_ext.test_asym_r8_is_parent_grid,
              lambda: pins_ext.test_asym_child_is_mean_of_parent_bucket(2),
              lambda: pins_ext.test_asym_qgemm_exact_rational_bruteforce(3),
              pins_ext.test_asym_qgemm_reduces_to_symmetric_and_is_linear_in_z,
              pins_ext.test_choose_single_width8_is_nearest_grid_point,
              pins_ext.test_choose_single_width4_takes_first_code_of_nearest_level,
              pins_ext.test_choose_exact_rational_bruteforce,
              pins_ext.test_choose_zero_weight_widths_drop_out,
              pins_ext.test_choose_all_zero_lambdas_tie_to_code_zero]
    return calls


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(mutant_c), "-o",
                    str(so), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._configure(ctypes.CDLL(str(so))))
    failures = 0
    for call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError):
            failures += 1
    assert failures > 0, f"mutant {name} passed every pin"
