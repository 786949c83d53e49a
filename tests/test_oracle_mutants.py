"""The oracle's pins must fail when a plausible mistake is planted in the oracle.

Each mutant is a copy of oracle/mpgemm_oracle.c with one edit (a flipped sign, a wrong
index, a dropped term, a transposed operand, a different rounding rule, a wrong layout
formula).  It is compiled into a temporary directory and the pin suite
(tests/test_oracle.py) runs against it in a subprocess; the suite must report failures.
Everything happens on the CPU; the real oracle library is never touched.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mpgemm_oracle.c")

MUTANTS = {
    "sign_of_q_minus_z": ("(double)(q - z) * s", "(double)(z - q) * s"),
    "group_index_mod": ("int grp = k / g;", "int grp = k % g;"),
    "zero_index": ("zeros[(size_t)grp * N + n] & 0xf", "zeros[(size_t)(n % (K / g)) * N + n] & 0xf"),
    "nibble_order_plain": ("(i % 2 == 0) ? i / 2 : 4 + i / 2", "i"),
    "lane_formula": ("int lane = nn + 16 * ((kk % 32) / 8);", "int lane = nn * 4 + ((kk % 32) / 8);"),
    "transposed_w": ("act_to_f64(w[(size_t)k * N + n], dtype)",
                     "act_to_f64(w[(size_t)(k % N) * N + (n % K)], dtype)"),
    "dropped_last_k": ("for (int k = 0; k < K; ++k) {\n                acc",
                       "for (int k = 0; k < K - 1; ++k) {\n                acc"),
    "round_half_up": ("double count = rint(a / spacing);",
                      "double count = floor(a / spacing + 0.5);"),
    "meta_reversed_in_strip": ("(size_t)(k / g) * 16 + (size_t)(n % 16);",
                               "(size_t)(k / g) * 16 + (size_t)(15 - n % 16);"),
}


# Mistakes in the 8-bit functions, caught by tests/test_oracle_w8.py.
MUTANTS_W8 = {
    "w8_sign": ("double d = (double)(q8 - z8);", "double d = (double)(z8 - q8);"),
    "w8_sym_zero": ("zeros[(size_t)r * N + n] : 128;", "zeros[(size_t)r * N + n] : 127;"),
    "w8_group_row": ("int r = k / g;                             /* group row of k */",
                     "int r = (k + 1) / g;"),
    "w8_step_bytes": ("(size_t)(kk / 32) * 8 + (size_t)(kk % 8);",
                      "(size_t)(kk / 32) + (size_t)(kk % 8) * 2;"),
    "w8_lane": ("int lane8 = col + 16 * ((kk % 32) / 8);", "int lane8 = col * 4 + ((kk % 32) / 8);"),
    "w8_zero_nibble": ("if (zeros) meta_zeros[e] = zeros[(size_t)r * N + n];",
                       "if (zeros) meta_zeros[e] = zeros[(size_t)r * N + n] & 0xf;"),
}


MUTANTS_FP8 = {
    "fp8_bias": ("ldexp((double)(8 + f), e - 10);", "ldexp((double)(8 + f), e - 11);"),
    "fp8_subnormal": ("ldexp((double)f, -9);", "ldexp((double)f, -10);"),
    "fp8_subnormal_implicit": ("ldexp((double)f, -9);", "ldexp((double)(8 + f), -9);"),
    "fp8_nan_all_exp15": ("if (e == 15 && f == 7) {", "if (e == 15 && f >= 6) {"),
    "fp8_sign": ("return sign ? -v : v;                          /* E4M3 sign bit */",
                 "return v;"),
    "fp8_mantissa_bits": ("int f = b & 0x7;", "int f = b & 0x3;"),
    "e5m2_bias": ("ldexp((double)(4 + fr), ex - 17);", "ldexp((double)(4 + fr), ex - 16);"),
    "e5m2_subnormal": ("ldexp((double)fr, -16);", "ldexp((double)fr, -15);"),
    "e5m2_inf_is_nan": ("v = fr ? NAN : INFINITY;", "v = NAN;"),
    "e5m2_sign": ("return neg ? -v : v;", "return v;"),
    "fp8_format_swap": ("format == 1 ? oracle_e5m2_to_f64(q)", "format == 0 ? oracle_e5m2_to_f64(q)"),
    "fp8_group_row": ("int row = k / g;", "int row = (k + 1) / g;"),
    "fp8_scale_col": ("scales[(size_t)row * N + n]", "scales[(size_t)row * N + (n ^ 1)]"),
}


MUTANTS_RAGGED = {
    "pad_k_to_256": ("(K + 127) / 128 * 128", "(K + 255) / 256 * 256"),
    "pad_n_to_32": ("(N + 15) / 16 * 16", "(N + 31) / 32 * 32"),
    "pad_code_zero_w4": ("(uint32_t)(zero_point(zeros, k / g, n, N, rows, 8) & 0xf)", "0u"),
    "pad_sym_zero_w8": ("(uint8_t)zero_point(zeros, k / g, n, N, rows, 128)",
                        "(uint8_t)zero_point(zeros, k / g, n, N, rows, 0)"),
    "pad_group_past_end": ("return r < rows ? zeros[(size_t)r * N + n] : 0;",
                           "return r < rows ? zeros[(size_t)r * N + n] : 8;"),
    "unpack_w8_unpadded": ("codes[(size_t)k * N + n] = packed_codes[code8_byte_offset(k, n, Kp)];",
                           "codes[(size_t)k * N + n] = packed_codes[code8_byte_offset(k, n, K)];"),
}


MUTANTS_LOWBIT = {
    "lowbit_sign": ("f64_to_act((double)(qb - zb) * sb, dtype);",
                    "f64_to_act((double)(zb - qb) * sb, dtype);"),
    "lowbit_sym_zero": ("(zeros[(size_t)gr * N + n] & cmask) : (1 << (bits - 1));",
                        "(zeros[(size_t)gr * N + n] & cmask) : (1 << bits) / 4;"),
    "lowbit_code_mask": ("int qb = codes[(size_t)k * N + n] & cmask;",
                         "int qb = codes[(size_t)k * N + n] & 0xf;"),
    "w2_field_order": ("bit = h + 2 * ((r % 8) % 4) + 8 * ((r % 8) / 4) + c;\n        } else if (r < 15) {\n            word = r / 5;\n            bit = h + 3 * (r % 5) + c;\n        } else {\n            word = c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)",
                       "bit = h + 2 * ((r % 8) / 2) + 8 * ((r % 8) % 2) + c;\n        } else if (r < 15) {\n            word = r / 5;\n            bit = h + 3 * (r % 5) + c;\n        } else {\n            word = c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)"),
    "w3_spare_pair": ("            word = c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)",
                      "            word = 2 - c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)"),
    "lowbit_tile_stride": ("uint8_t *lane_words = plane + T * 256 * bits + (size_t)L * 4 * bits;\n    for (int c = 0; c < bits; ++c) {\n        int word, bit;\n        if (bits == 2) {\n            word = r / 8;\n            bit = h + 2 * ((r % 8) % 4) + 8 * ((r % 8) / 4) + c;\n        } else if (r < 15) {\n            word = r / 5;\n            bit = h + 3 * (r % 5) + c;\n        } else {\n            word = c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)",
                           "uint8_t *lane_words = plane + T * 256 * bits + (size_t)(L ^ 16) * 4 * bits;\n    for (int c = 0; c < bits; ++c) {\n        int word, bit;\n        if (bits == 2) {\n            word = r / 8;\n            bit = h + 2 * ((r % 8) % 4) + 8 * ((r % 8) / 4) + c;\n        } else if (r < 15) {\n            word = r / 5;\n            bit = h + 3 * (r % 5) + c;\n        } else {\n            word = c;\n            bit = h + 15;\n        }\n        if ((q >> c) & 1u)"),
    "lowbit_pad_zero": ("(uint32_t)zero_point(zeros, k / g, n, N, rows, 1 << (bits - 1));",
                        "(uint32_t)zero_point(zeros, k / g, n, N, rows, 0);"),
}


MUTANTS_ATTENTION = {
    "gqa_head_modulo": ("const int hk = h / group;\n            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;\n            double mx = -INFINITY;\n            for (int t = 0; t < len; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double s_k",
                        "const int hk = h % Hkv;\n            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;\n            double mx = -INFINITY;\n            for (int t = 0; t < len; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double s_k"),
    "no_softmax_scale": ("dot += act_to_f64(qh[d], dtype) * kd;\n                }\n                score[t] = dot * (double)scale;",
                         "dot += act_to_f64(qh[d], dtype) * kd;\n                }\n                score[t] = dot;"),
    "kvfp8_gqa_head_modulo": ("const int hk = h / group;\n            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;\n            double mx = -INFINITY;\n            for (int t = 0; t < len; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double sk8",
                              "const int hk = h % Hkv;\n            const uint16_t *qh = q + ((size_t)b * Hq + h) * D;\n            double mx = -INFINITY;\n            for (int t = 0; t < len; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double sk8"),
    "k_zero_sign": ("f64_to_act((double)((int)kc[row * D + d] - (int)kz[row]) * s_k, dtype)",
                    "f64_to_act((double)((int)kz[row] - (int)kc[row * D + d]) * s_k, dtype)"),
    "v_takes_k_scale": ("const double s_v = oracle_f16_to_f64(vs[row]);",
                        "const double s_v = oracle_f16_to_f64(ks[row]);"),
    "v_not_rounded": ("double vd = act_to_f64(\n                        f64_to_act((double)((int)vc[row * D + d] - (int)vz[row]) * s_v, dtype), dtype);",
                      "double vd = (double)((int)vc[row * D + d] - (int)vz[row]) * s_v;"),
    "last_token_dropped": ("            for (int t = 0; t < len; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double s_v",
                           "            for (int t = 0; t < len - 1; ++t) {\n                const size_t row = ((size_t)b * Tmax + t) * Hkv + hk;\n                const double s_v"),
    "kv_v_not_transposed": ("hb[64 * Dp + code8_byte_offset(slot, d, 64)] = d < D ? vc[row * D + d] : 0;",
                            "hb[64 * Dp + code8_byte_offset(d, slot, (int)Dp)] = d < D ? vc[row * D + d] : 0;"),
    "kv_zeros_swapped": ("hb[128 * Dp + 256 + slot] = kz[row];",
                         "hb[128 * Dp + 320 + slot] = kz[row];"),
    "kv_pad_not_zero": ("hb[code8_byte_offset(d, slot, (int)Dp)] = d < D ? kc[row * D + d] : 0;",
                        "hb[code8_byte_offset(d, slot, (int)Dp)] = d < D ? kc[row * D + d] : 128;"),
    "kv_unpadded_head": ("static size_t kv_padded_d(int D) { return (size_t)(D + 63) / 64 * 64; }",
                         "static size_t kv_padded_d(int D) { return (size_t)(D + 15) / 16 * 16; }"),
    "kvfp8_format_swap": ("double e8 = format == 1 ? oracle_e5m2_to_f64(c8) : oracle_e4m3_to_f64(c8);\n                    acc[d]",
                          "double e8 = format == 0 ? oracle_e5m2_to_f64(c8) : oracle_e4m3_to_f64(c8);\n                    acc[d]"),
    "kvfp8_v_scale": ("const double sv8 = oracle_f16_to_f64(vs[row]);",
                      "const double sv8 = oracle_f16_to_f64(ks[row]);"),
    "kvfp8_k_unrounded": ("dot += act_to_f64(qh[d], dtype) * act_to_f64(f64_to_act(e8 * sk8, dtype), dtype);",
                          "dot += act_to_f64(qh[d], dtype) * e8 * sk8;"),
}


def _run_pins(text, before, after, pins, tmp_path):
    assert text.count(before) == 1, f"mutation anchor not found once: {before}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(before, after))
    lib = oracle.build(src=str(src), out=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, MPGEMM_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pins)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(MUTANTS_W8))
def test_w8_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS_W8[name]
    res = _run_pins(open(SRC).read(), before, after, "test_oracle_w8.py", tmp_path)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation anchor for {name} not found once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(before, after))
    lib = oracle.build(src=str(src), out=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, MPGEMM_ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_FP8))
def test_fp8_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS_FP8[name]
    res = _run_pins(open(SRC).read(), before, after, "test_oracle_fp8.py", tmp_path)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_RAGGED))
def test_ragged_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS_RAGGED[name]
    res = _run_pins(open(SRC).read(), before, after, "test_oracle_ragged.py", tmp_path)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_LOWBIT))
def test_lowbit_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS_LOWBIT[name]
    res = _run_pins(open(SRC).read(), before, after, "test_oracle_lowbit.py", tmp_path)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_ATTENTION))
def test_attention_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS_ATTENTION[name]
    res = _run_pins(open(SRC).read(), before, after, "test_oracle_attention.py", tmp_path)
    assert res.returncode == 1, f"pins did not catch mutant {name}:\n{res.stdout[-2000:]}"
