"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins in test_oracle_pins.py catch every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "rms_divides_by_head_dim": ("ss / (channels > 0 ? channels : (double)C) + eps",
                                "ss / (channels > 0 ? channels : (double)d) + eps"),
    "eps_outside_sqrt": ("1.0 / sqrt(ss / (channels > 0 ? channels : (double)C) + eps)",
                         "1.0 / (sqrt(ss / (channels > 0 ? channels : (double)C)) + eps)"),
    "gamma_dropped": ("y[c] = load(dtype, x, x0 + c) * inv_rms * load(dtype, gamma, c);",
                      "y[c] = load(dtype, x, x0 + c) * inv_rms;"),
    "rotate_half_sign": ("(i < h2) ? -yh[i + h2] : yh[i - h2]", "(i < h2) ? yh[i + h2] : -yh[i - h2]"),
    "rotate_half_partner": ("(i < h2) ? -yh[i + h2] : yh[i - h2]", "(i < h2) ? -yh[h2 - 1 - i] : yh[d - 1 - i]"),
    "cos_half_index": ("yh[i] * load(dtype, cs, r0 + i)", "yh[i] * load(dtype, cs, r0 + i % h2)"),
    "interleave_not_deinterleaved": ("double p1 = j < half ? z[2 * j] : z[2 * (j - half) + 1];",
                                     "double p1 = z[j];"),
    "interleave_sign": ("double p2 = j < half ? -z[2 * j + 1] : z[2 * (j - half)];",
                        "double p2 = j < half ? z[2 * j + 1] : -z[2 * (j - half)];"),
    "v2_rope_on_raw_kv": ("z[i] = v2 ? y[i] :", "z[i] = v2 ? load(in_dtype, kv, kv0 + i) :"),
    "v1_rms_over_whole_row": ("for (int64_t i = 0; i < rms_size; i++) {\n                double xi",
                              "for (int64_t i = 0; i < Dkv; i++) {\n                double xi"),
    "pa_head_major_layout": ("int64_t r = (blk * block_size + off) * N + n;",
                             "int64_t r = (blk * N + n) * block_size + off;"),
    "norm_ignores_batch": ("int64_t r = (b * N + n) * cache_dim0 + slot;", "int64_t r = n * cache_dim0 + slot;"),
    "round_half_up": ("double r = nearbyint(t);", "double r = floor(t + 0.5);"),
    "offset_before_scale": ("    if (scale) t = t * scale[qi];\n    if (offset) t = t + offset[qi];",
                            "    if (offset) t = t + offset[qi];\n    if (scale) t = t * scale[qi];"),
    "e4m3_no_saturation": ("if (a >= 448.0) return s | 0x7E;", "if (a >= 464.0) return s | 0x7F;"),
    "bf16_truncates": ("return nearbyint(a / q) * q;", "return floor(a / q) * q;"),
    "e5m2_no_saturation": ("if (a >= 57344.0) return s | 0x7B;", "if (a >= 61440.0) return s | 0x7C;"),
    "e5m2_wrong_bias": ("return s | (uint8_t)((E + 15) << 2) | mant;", "return s | (uint8_t)((E + 16) << 2) | mant;"),
    "pa_blk_start_not_offset": ("slot = start < 0 ? -1 : start + s % block_size;", "slot = start;"),
    "pa_blk_per_token_index": ("int64_t start = index[b * nblk + s / block_size];",
                               "int64_t start = index[(b * S + s) / block_size];"),
    "no_capacity_check": ("if (slot >= 0 && slot < capacity) {", "if (slot >= 0) {"),
    "per_head_denominator": ("double inv_rms = 1.0 / sqrt(ss / (double)d + eps);",
                             "double inv_rms = 1.0 / sqrt(ss / (double)(nh * d) + eps);"),
    "per_head_gamma_dropped": ("y[h * d + i] = load(dtype, x, x0 + h * d + i) * inv_rms * load(dtype, gamma, i);",
                               "y[h * d + i] = load(dtype, x, x0 + h * d + i) * inv_rms;"),
    "split_ignores_given_sum": ("            ss = *given_ss;\n", "            ss = 0.0 * *given_ss + 1.0;\n"),
    "split_ignores_total_channels": ("ss / (channels > 0 ? channels : (double)C) + eps",
                                     "ss / (double)C + eps"),
    "sumsq_not_squared": ("            double v = load(dtype, x, t * n * d + c);\n            ss += v * v;",
                          "            double v = load(dtype, x, t * n * d + c);\n            ss += fabs(v);"),
    "linear_weight_transposed": ("acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);",
                                 "acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, (h * I + i) % (I * H));"),
    "linear_bias_dropped": ("acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);\n"
                            "            if (a_scale) acc *= a_scale[s];\n"
                            "            if (w_scale) acc *= w_scale[i];\n"
                            "            if (bias) acc += load(bias_dtype, bias, i);\n",
                            "acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);\n"
                            "            if (a_scale) acc *= a_scale[s];\n"
                            "            if (w_scale) acc *= w_scale[i];\n"),
    "linear_weight_scale_dropped": ("acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);\n"
                                    "            if (a_scale) acc *= a_scale[s];\n"
                                    "            if (w_scale) acc *= w_scale[i];\n",
                                    "acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);\n"
                                    "            if (a_scale) acc *= a_scale[s];\n"),
    "mx_weight_block_scale_ignored": ("* dec_e8m0(w_bs[i * w_bs_stride + h / 32]);", "* 1.0;"),
    "mx_e8m0_bias_128": ("return e == 255 ? NAN : ldexp(1.0, (int)e - 127);",
                         "return e == 255 ? NAN : ldexp(1.0, (int)e - 128);"),
    "mx_first_block_scale_for_every_block": ("a_bs[s * a_bs_stride + h / 32]", "a_bs[s * a_bs_stride]"),
    "c_kv_from_raw_in_v1": ("c_src[i] = v2 ? load(in_dtype, v, row * Dv + i) : y[i];",
                            "c_src[i] = v2 ? load(in_dtype, v, row * Dv + i) : load(in_dtype, kv, kv0 + i);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", str(mutant), "-o", str(lib), "-lm"])
    env = dict(os.environ, QKNR_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
