"""Planted mistakes in the oracle must be caught by its pins.

Each case compiles a copy of ``oracle/oracle.c`` with one plausible slip (a
dropped term, a wrong sign or index, a transposed operand, a different
rounding rule) into a temporary library, runs ``test_oracle_pins.py``
against it in a subprocess, and requires that run to fail. CPU only.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "round_after_adding_z": ("float r = rintf(x[j] / s) + z;", "float r = rintf(x[j] / s + z);"),
    "round_half_away": ("float r = rintf(x[j] / s);", "float r = roundf(x[j] / s);"),
    "asym_levels_2^b": ("const float s = range / qmaxu;", "const float s = range / (qmaxu + 1.0f);"),
    "sym_qmax_2^(b-1)": ("const float qmax = (float)((1 << (bits - 1)) - 1);",
                         "const float qmax = (float)(1 << (bits - 1));"),
    "zero_point_sign": ("const float z = rintf(-mn / s) + 0.0f;", "const float z = rintf(mn / s) + 0.0f;"),
    "no_range_floor": ("if (range < ORACLE_FLOOR) range = ORACLE_FLOOR;", ";"),
    "nibble_order_swapped": ("row_codes[j / 2] = (uint8_t)((u0 & 0xFu) | ((u1 & 0xFu) << 4));",
                             "row_codes[j / 2] = (uint8_t)((u1 & 0xFu) | ((u0 & 0xFu) << 4));"),
    "sym_offset_7": ("uint32_t u0 = (uint32_t)(symmetric ? q[j] + 8 : q[j]);",
                     "uint32_t u0 = (uint32_t)(symmetric ? q[j] + 7 : q[j]);"),
    "dequant_plus_z": ("out[r * k + j] = (qf - z) * s;", "out[r * k + j] = (qf + z) * s;"),
    "matmul_transposed_x": ("acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)wrow[j];",
                            "acc += (double)bf16_bits_to_f32(x[j * m + i < m * k ? j * m + i : 0]) * (double)wrow[j];"),
    "matmul_drops_last_element": ("for (int64_t j = 0; j < k; ++j)\n                acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)wrow[j];",
                                  "for (int64_t j = 0; j + 1 < k; ++j)\n                acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)wrow[j];"),
    "int8_row_stride_halved": ("const int64_t codes_per_row = bits == 4 ? k / 2 : k;",
                               "const int64_t codes_per_row = k / 2;"),
    "int8_sym_read_unsigned": ("return symmetric ? (int32_t)(int8_t)row_codes[j] : (int32_t)row_codes[j];",
                               "return (int32_t)row_codes[j];"),
    "awq_grid_misses_one": ("const float alpha = (float)i / (float)n_grid;",
                            "const float alpha = (float)i / (float)(n_grid + 1);"),
    "awq_channel_max_not_mean": ("for (int64_t i = 0; i < t; ++i) acc += fabs((double)bf16_bits_to_f32(x[i * k + j]));",
                                 "for (int64_t i = 0; i < t; ++i) acc = fmax(acc, (double)t * fabs((double)bf16_bits_to_f32(x[i * k + j])));"),
    "awq_activation_times_s": ("f32_to_bf16_rne(bf16_bits_to_f32(x[i * k + j]) / s[j])",
                               "f32_to_bf16_rne(bf16_bits_to_f32(x[i * k + j]) * s[j])"),
    "awq_weights_unscaled": ("if (oracle_quantize_bf16(w, n, k, bits, symmetric, group, s, codes, sc, zr)) goto out;",
                             "if (oracle_quantize_bf16(w, n, k, bits, symmetric, group, NULL, codes, sc, zr)) goto out;"),
    "awq_argmax": ("if (losses[i] < losses[arg]) arg = i;", "if (losses[i] > losses[arg]) arg = i;"),
    "awq_abs_error": ("total += d * d;", "total += fabs(d);"),
    "mx_ties_to_odd": ("if (d < db || (d == db && (i & 1) == 0)) best = i;",
                       "if (d < db || (d == db && (i & 1) == 1)) best = i;"),
    "mx_scale_floor_clips": ("int e = p - 3 + (m > 0.75f ? 1 : 0);", "int e = p - 3;"),
    "mx_nibble_order": ("codes[r * (k / 2) + b * 16 + j / 2] = (uint8_t)(nib[j] | (nib[j + 1] << 4));",
                        "codes[r * (k / 2) + b * 16 + j / 2] = (uint8_t)(nib[j + 1] | (nib[j] << 4));"),
    "mx_negative_zero_kept": ("nib[j] = (uint8_t)(mag == 0 ? 0 : ((v < 0.0f ? 8 : 0) | mag));",
                              "nib[j] = (uint8_t)((v < 0.0f ? 8 : 0) | mag);"),
    "gptq_update_sign": ("for (int64_t f = j + 1; f < k; ++f) row[f] = fmaf(-d, u[j * k + f], row[f]);",
                         "for (int64_t f = j + 1; f < k; ++f) row[f] = fmaf(d, u[j * k + f], row[f]);"),
    "gptq_error_not_scaled": ("const float d = (row[j] - w_hat) / u[j * k + j];", "const float d = (row[j] - w_hat);"),
    "gptq_updates_stay_in_group": ("for (int64_t f = j + 1; f < k; ++f) row[f] = fmaf(-d, u[j * k + f], row[f]);",
                                   "for (int64_t f = j + 1; f < (j / group + 1) * group; ++f) row[f] = fmaf(-d, u[j * k + f], row[f]);"),
    "gptq_absolute_damping": ("for (int64_t i = 0; i < k; ++i) h[i * k + i] += percdamp * mean;",
                              "for (int64_t i = 0; i < k; ++i) h[i * k + i] += percdamp;"),
    "gptq_hessian_without_2": ("h[i * k + j] = h[j * k + i] = 2.0 * acc;", "h[i * k + j] = h[j * k + i] = acc;"),
    "smooth_inverted": ("s[j] = sqrtf(a) / sqrtf(b);", "s[j] = sqrtf(b) / sqrtf(a);"),
    "smooth_alpha_swapped": ("s[j] = powf(a, alpha) / powf(b, 1.0f - alpha);",
                             "s[j] = powf(a, 1.0f - alpha) / powf(b, alpha);"),
    "activation_times_smooth": ("row[j] = smooth ? v / smooth[j] : v;", "row[j] = smooth ? v * smooth[j] : v;"),
    "weight_axis_max_over_k": ("float v = fabsf(bf16_bits_to_f32(w[r * k + j]));\n            if (v > aw[j]) aw[j] = v;",
                               "float v = fabsf(bf16_bits_to_f32(w[r * k + j]));\n            if (v > aw[r % k]) aw[r % k] = v;"),
    "per_token_qmax_255": ("const float s = a / 127.0f;", "const float s = a / 255.0f;"),
    "w8a8_drops_weight_scale": ("y[i * n + r] = (double)a * (double)sx[i] * (double)sw[r];",
                                "y[i * n + r] = (double)a * (double)sx[i];"),
    "effective_bits_zero_dropped": ("(double)(scale_bits + zero_bits) / (double)group",
                                    "(double)(scale_bits) / (double)group"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut_c = tmp_path / "oracle_mut.c"
    mut_c.write_text(src.replace(old, new))
    mut_so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", str(mut_c), "-o", str(mut_so), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(mut_so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
