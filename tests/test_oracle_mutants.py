"""Plausible mistakes planted in a copy of the oracle must fail a pin.

Each mutant is a one-line edit of ``oracle/snr_oracle.c`` compiled into a
temporary library; the pins of ``oracle_pins.py`` are run against it and at
least one of them must fail. This shows the pins can go red for each class of
error (epsilon placement, divisor, dropped tail elements, dropped gain, sign
of the residual add, which epsilon and which gain each norm of the tail uses,
the row stride, the bf16 decode, f32 accumulation, a skipped element, a
missing root, and the Q8_1 block rules). CPU only: the mistakes are planted in the
oracle, never in GPU code.
"""
import os

import pytest

import oracle as oracle_pkg
from oracle_pins import ALL_PINS

MUTANTS = {
    "eps_outside_root": ("const double rms = sqrt(mean_sq + eps);",
                         "const double rms = sqrt(mean_sq) + eps;"),
    "eps_added_to_sum": ("const double mean_sq = sum_sq / (double)n;",
                         "const double mean_sq = (sum_sq + eps) / (double)n - eps;"),
    "divide_by_n_minus_1": ("const double mean_sq = sum_sq / (double)n;",
                            "const double mean_sq = sum_sq / (double)(n > 1 ? n - 1 : 1);"),
    "drop_ragged_tail": ("    for (int64_t j = 0; j < n; ++j)\n        sum_sq += x[j] * x[j];",
                         "    for (int64_t j = 0; j < (n & ~(int64_t)3); ++j)\n        sum_sq += x[j] * x[j];"),
    "sum_abs_not_squares": ("sum_sq += x[j] * x[j];", "sum_sq += fabs(x[j]);"),
    "sum_in_float": ("double sum_sq = 0.0;", "float sum_sq = 0.0f;"),
    "sum_skips_first": ("    for (int64_t j = 0; j < n; ++j)\n        sum_sq += x[j] * x[j];",
                        "    for (int64_t j = 1; j < n; ++j)\n        sum_sq += x[j] * x[j];"),
    "rms_without_root": ("const double rms = sqrt(mean_sq + eps);",
                         "const double rms = mean_sq + eps;"),
    "drop_gain": ("y[j] = x[j] / rms * gamma[j];", "y[j] = x[j] / rms;"),
    "multiply_by_rms": ("y[j] = x[j] / rms * gamma[j];", "y[j] = x[j] * rms * gamma[j];"),
    "residual_sign": ("hi[j] = (double)r[i * n + j] + p[j];",
                      "hi[j] = (double)r[i * n + j] - p[j];"),
    "residual_dropped": ("hi[j] = (double)r[i * n + j] + p[j];", "hi[j] = p[j];"),
    "post_norm_uses_pre_eps": ("rms_row(ar, gp, (double)eps_post, n, p)",
                               "rms_row(ar, gp, (double)eps_pre, n, p)"),
    "pre_norm_uses_post_eps": ("rms_row(hi, gq, (double)eps_pre, n, y + i * n)",
                               "rms_row(hi, gq, (double)eps_post, n, y + i * n)"),
    "second_norm_on_p": ("rms_row(hi, gq, (double)eps_pre, n, y + i * n)",
                         "rms_row(p, gq, (double)eps_pre, n, y + i * n)"),
    "gains_swapped": ("rms_row(ar, gp, (double)eps_post, n, p)",
                      "rms_row(ar, gq, (double)eps_post, n, p)"),
    "row_stride_lost": ("xr[j] = (double)x[i * n + j];", "xr[j] = (double)x[j];"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)b << 16;",
                          "uint32_t u = (uint32_t)b << 15;"),
    "bf16_gamma_as_one": ("gr[j] = (double)bf16_bits_to_f32(gamma[j]);",
                          "gr[j] = 1.0;"),
    "scale_only_on_norm": ("oi[j] = (oi[j] + (double)r[i * n + j]) * scale;",
                           "oi[j] = oi[j] * scale + (double)r[i * n + j];"),
    "norm_add_subtracts": ("oi[j] = (oi[j] + (double)r[i * n + j]) * scale;",
                           "oi[j] = (oi[j] - (double)r[i * n + j]) * scale;"),
    "add_norm_subtracts": ("si[j] = (double)a[i * n + j] + (double)b[i * n + j];",
                           "si[j] = (double)a[i * n + j] - (double)b[i * n + j];"),
    "add_norm_drops_b": ("si[j] = (double)a[i * n + j] + (double)b[i * n + j];",
                         "si[j] = (double)a[i * n + j];"),
    "q8_divides_by_128": ("const double db = amax / 127.0;",
                          "const double db = amax / 128.0;"),
    "q8_truncates": ("double r = nearbyint(t[j]);", "double r = trunc(t[j]);"),
    "q8_rounds_half_away": ("double r = nearbyint(t[j]);",
                            "double r = round(t[j]);"),
    "q8_row_amax": ("if (fabs(yi[b * 32 + l]) > amax)\n                    amax = fabs(yi[b * 32 + l]);",
                    "if (fabs(yi[l]) > amax)\n                    amax = fabs(yi[l]);"),
    "q8_before_gain": ("t[j] = yi[b * 32 + l] / db;",
                       "t[j] = yi[b * 32 + l] / gr[b * 32 + l] / db;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle_pkg.SOURCE) as fh:
        src = fh.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle_pkg.build(str(mutated), str(tmp_path / "libmutant.so"))
    mutant = oracle_pkg.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # a pin that raises has caught the mutant
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
