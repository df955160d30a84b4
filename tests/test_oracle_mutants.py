"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/oracle.c`` (a dropped term,
a wrong rounding mode, a wrong sign or index, a transposed operand), builds it
on the CPU, and runs the oracle pin suites against that build in a
subprocess.  The pins must fail for every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_absmean.py"),
        os.path.join(ROOT, "tests", "test_oracle_act_linear.py"),
        os.path.join(ROOT, "tests", "test_oracle_glu.py"),
        os.path.join(ROOT, "tests", "test_oracle_backward.py"),
        os.path.join(ROOT, "tests", "test_oracle_b3.py")]

MUTANTS = {
    "ternarize_round_half_away": ("float r = rintf(scaled);", "float r = roundf(scaled);"),
    "ternarize_drops_eps": ("float denom = gamma + eps;", "float denom = gamma;"),
    "ternarize_no_clamp": ("if (r > 1.0f) r = 1.0f;", ""),
    "absmean_wrong_count": ("return round_ratio_to_f32(&total, (uint64_t)count);",
                            "return round_ratio_to_f32(&total, (uint64_t)count + 1);"),
    "absmean_drops_subnormal_scale": ("*shift = (int)biased - 1;", "*shift = (int)biased;"),
    "absmean_tie_to_odd": ("return (lo_bits & 1u) ? hi : lo;", "return (lo_bits & 1u) ? lo : hi;"),
    "pack_transposed_in_row": ("*byte = tile_start + r * 16 + t % 16;\n    *bit = 2 * (t / 16);",
                               "*byte = tile_start + r * 16 + t / 4;\n    *bit = 2 * (t % 4);"),
    "pack_row_major_tiles": ("int64_t tile_start = (tile_row * tiles_per_row + tile_col) * 256;",
                             "int64_t tile_start = (tile_col * ((k + 63) / 64) + tile_row) * 256;"),
    "quant_scale_128": ("float scale = 127.0f / (amax > 1e-5f ? amax : 1e-5f);",
                        "float scale = 128.0f / (amax > 1e-5f ? amax : 1e-5f);"),
    "quant_round_half_away": ("float r = rintf(prod);", "float r = roundf(prod);"),
    "quant_no_eps_floor": ("float scale = 127.0f / (amax > 1e-5f ? amax : 1e-5f);",
                           "float scale = 127.0f / (amax > 0.0f ? amax : 1.0f);"),
    "linear_sign_flip": ("for (int64_t t = 0; t < k; ++t) s += (int64_t)qx[i * k + t] * (int64_t)qw[j * k + t];",
                         "for (int64_t t = 0; t < k; ++t) s -= (int64_t)qx[i * k + t] * (int64_t)qw[j * k + t];"),
    "linear_transposed_operand": ("for (int64_t t = 0; t < k; ++t) s += (int64_t)qx[i * k + t] * (int64_t)qw[j * k + t];",
                                  "for (int64_t t = 0; t < k; ++t) s += (int64_t)qx[i * k + t] * (int64_t)qw[(t % n) * k + j % k];"),
    "rescale_drops_alpha": ("(double)acc[i * n + j] * (double)gamma * (double)alpha[i] / 127.0;",
                            "(double)acc[i * n + j] * (double)gamma / 127.0;"),
    "rescale_128": ("(double)acc[i * n + j] * (double)gamma * (double)alpha[i] / 127.0;",
                    "(double)acc[i * n + j] * (double)gamma * (double)alpha[i] / 128.0;"),
    "bf16_round_half_away": ("double r = nearbyint(ldexp(a, -ulp_exp));", "double r = round(ldexp(a, -ulp_exp));"),
    "glu_no_relu": ("double r = g > 0.0 ? g : 0.0;", "double r = g;"),
    "glu_not_squared": ("h[i * f + j] = orc_bf16_from_double(r * r * u);",
                        "h[i * f + j] = orc_bf16_from_double(r * u);"),
    "glu_halves_swapped": ("return (tile % 2 == 0 ? 0 : f) + 16 * (tile / 2) + r;",
                           "return (tile % 2 == 0 ? f : 0) + 16 * (tile / 2) + r;"),
    "glu_up_from_gate_row": ("double u = (double)acc[i * 2 * f + f + j] * s;",
                             "double u = (double)acc[i * 2 * f + j] * s;"),
    "backward_x_no_gamma": ("dx[i * k + t] = (float)((double)gamma * s);", "dx[i * k + t] = (float)s;"),
    "backward_x_untransposed": ("                trit_position(j, t, k, &byte, &bit);\n                int w = (int)((packed[byte] >> bit) & 3u) - 1;\n                s += (double)w * bf16_to_double(dy[i * n + j]);",
                                "                trit_position(t % n, j % k, k, &byte, &bit);\n                int w = (int)((packed[byte] >> bit) & 3u) - 1;\n                s += (double)w * bf16_to_double(dy[i * n + j]);"),
    "backward_w_no_alpha": ("s += bf16_to_double(dy[i * n + j]) * (double)alpha[i] * (double)qx[i * k + t];",
                            "s += bf16_to_double(dy[i * n + j]) * (double)qx[i * k + t];"),
    "backward_w_128": ("dw[j * k + t] = (float)(s / 127.0);", "dw[j * k + t] = (float)(s / 128.0);"),
    "pack_transposed_not_transposed": ("for (int64_t t = 0; t < k; ++t) qt[t * n + j] = q[j * k + t];",
                                       "for (int64_t t = 0; t < k; ++t) qt[j * k + t] = q[j * k + t];"),
    "b3_floor_encoding": ("return (uint8_t)((256 * v + 242) / 243);", "return (uint8_t)((256 * v) / 243);"),
    "b3_digit_order_reversed": ("*digit = (int)(u / 16);", "*digit = 4 - (int)(u / 16);"),
    "b3_group_row_swapped": ("g * 256 + (row % 16) * 16 + u % 16;", "(row % 16) * 64 + g * 16 + u % 16;"),
    "b3_padding_not_zero": ("memset(trits, 0, (size_t)(5 * total));     /* padding: trit 0 */",
                            "memset(trits, 1, (size_t)(5 * total));     /* padding: trit 0 */"),
    "b3_forward_digit_off_by_one": ("s += (int64_t)t[digit] * xq[i * k + c];",
                                    "s += (int64_t)t[(digit + 1) % 5] * xq[i * k + c];"),
    "unpack_codes_not_trits": ("q[row * k + col] = (int8_t)((int)((packed[byte] >> bit) & 3u) - 1);",
                               "q[row * k + col] = (int8_t)((int)((packed[byte] >> bit) & 3u));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mutant_c), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, BITLINEAR_ORACLE_SO=str(so), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"
