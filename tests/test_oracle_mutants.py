"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant is oracle.c with one deliberate error: a wrong rounding rule, a
dropped term, a flipped sign, a wrong index or a transposed operand.  The
mutant is compiled to a temporary library and the pin suites are run against
it in a subprocess; every mutant must make at least one pin fail.  Mutants are
chosen so that none writes outside its buffers.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_codec.py"),
        os.path.join(ROOT, "tests", "test_oracle_attention.py"),
        os.path.join(ROOT, "tests", "test_oracle_per_head.py"),
        os.path.join(ROOT, "tests", "test_oracle_prefill.py"),
        os.path.join(ROOT, "tests", "test_oracle_rotation.py"),
        os.path.join(ROOT, "tests", "test_oracle_codecs.py")]

MUTANTS = {
    "subnormal_ties_away": ("double m = rint(a * 512.0);", "double m = round(a * 512.0);"),
    "normal_ties_up": ("double m = rint((ldexp(a, -e) - 1.0) * 8.0);",
                       "double m = floor((ldexp(a, -e) - 1.0) * 8.0 + 0.5);"),
    "saturate_to_nan": ("if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
                        "if (a >= 448.0) return (uint8_t)(sign | 0x7F);"),
    "no_saturation_above_448": ("if (a >= 448.0) return", "if (a >= 480.0) return"),
    "subnormal_step": ("mag = ldexp((double)M, -9);", "mag = ldexp((double)M, -8);"),
    "exponent_bias": ("mag = ldexp(1.0 + (double)M / 8.0, E - 7);",
                      "mag = ldexp(1.0 + (double)M / 8.0, E - 8);"),
    "nan_loses_sign": ("if (isnan(y)) return (uint8_t)(sign | 0x7F);",
                       "if (isnan(y)) return (uint8_t)0x7F;"),
    "reciprocal_multiply": ("float y = x / scale;", "float y = x * (1.0f / scale);"),
    "bf16_bits_misplaced": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "no_softmax_scale": ("s[j] = dot / sqrt((double)D);", "s[j] = dot;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no_normalisation": ("for (int i = 0; i < D; ++i) out[i] /= Z;", "(void)Z;"),
    "value_tile_token_major": (
        "return ((blk * Hkv + h) * (int64_t)D + i) * (int64_t)bs + off;",
        "return ((blk * Hkv + h) * (int64_t)bs + off) * (int64_t)D + i;"),
    "key_tile_token_major": (
        "int64_t byte_in_tile = ((int64_t)((off / 4) * C + c) * 4 + off % 4) * (4 * K) + g * K + w % K;",
        "int64_t byte_in_tile = ((int64_t)off * D + i) * eb;"),
    "key_tile_quarters_swapped": (
        "int g = i / q;                     /* quarter */",
        "int g = (3 - i / q);               /* quarter */"),
    "gqa_interleaved_heads": ("int h = hq / g;", "int h = hq % Hkv;"),
    "window_off_by_one": ("? L - window : 0;", "? L - window + 1 : 0;"),
    "slot_offset_shift": ("int off = (int)(j % bs);", "int off = (int)((j + 1) % bs);"),
    "k_scale_for_values": ("((uint8_t*)value_cache)[vi] = oracle_quantize(xv, v_scale);",
                           "((uint8_t*)value_cache)[vi] = oracle_quantize(xv, k_scale);"),
    "scale_dropped_in_decode": ("return oracle_e4m3_decode(((const uint8_t*)cache)[idx]) * scale;",
                                "return oracle_e4m3_decode(((const uint8_t*)cache)[idx]);"),
    "bf16_cache_bits_altered": (
        "oracle_quantize(xv, v_scale);\n                } else {\n                    ((uint16_t*)key_cache)[ki] = xk;",
        "oracle_quantize(xv, v_scale);\n                } else {\n                    ((uint16_t*)key_cache)[ki] = (uint16_t)(xk ^ 0x0001);"),
    "per_head_write_head0_scale": ("((uint8_t*)key_cache)[ki] = oracle_quantize(xk, k_scales[h]);",
                                   "((uint8_t*)key_cache)[ki] = oracle_quantize(xk, k_scales[0]);"),
    "per_head_values_with_key_scales": ("((uint8_t*)value_cache)[vi] = oracle_quantize(xv, v_scales[h]);",
                                        "((uint8_t*)value_cache)[vi] = oracle_quantize(xv, k_scales[h]);"),
    "per_head_decode_interleaved_heads": ("int kv = pairs[2 * p + 1] / g;",
                                          "int kv = pairs[2 * p + 1] % Hkv;"),
    "prefill_excludes_own_position": ("int64_t end = pos + 1;", "int64_t end = pos;"),
    "prefill_chunk_at_context_start": (
        "int64_t pos = (int64_t)context_lens[b] - chunk + (row - qsl[b]);",
        "int64_t pos = (row - qsl[b]);"),
    "prefill_first_query_row_for_all": (
        "qv[i] = (double)oracle_bf16_to_f32(q[(row * Hq + hq) * D + i]);",
        "qv[i] = (double)oracle_bf16_to_f32(q[((int64_t)qsl[b] * Hq + hq) * D + i]);"),
    "prefill_interleaved_kv_heads": ("int kvh = hq / group;", "int kvh = hq % Hkv;"),
    "prefill_window_off_by_one": ("? end - window : 0;", "? end - window + 1 : 0;"),
    "rotation_unnormalised": ("float c = (float)(1.0 / sqrt((double)d));", "float c = 1.0f;"),
    "rotation_f32_butterfly_sign": ("x[j + h] = a - b;", "x[j + h] = b - a;"),
    "rotation_f64_butterfly_sign": ("x[j + h] = -b + a;", "x[j + h] = b - a;"),
    "rotated_decode_output_not_rotated_back": (
        "oracle_hadamard_f64(o, D);              /* back to the original coordinates */",
        "(void)o;"),
    "rotated_decode_query_not_rotated": ("oracle_hadamard_f64(qr, D);", "(void)qr;"),
    "rotated_write_values_unrotated": ("oracle_hadamard_f32(rv, D);", "(void)rv;"),
    "rotated_per_head_write_head0_scale": ("quantize_f32(rk[i], k_scales ? k_scales[h] : k_scale)",
                                           "quantize_f32(rk[i], k_scales ? k_scales[0] : k_scale)"),
    "rotated_per_head_values_with_key_scales": (
        "quantize_f32(rv[i], v_scales ? v_scales[h] : v_scale)",
        "quantize_f32(rv[i], k_scales ? k_scales[h] : v_scale)"),
    "rotated_per_head_decode_interleaved_heads": ("int kvh = pairs[2 * p + 1] / group;",
                                                  "int kvh = pairs[2 * p + 1] % Hkv;"),
    "rotated_prefill_query_not_rotated": ("if (rotate) oracle_hadamard_f64(qv, D);", "(void)rotate;"),
    "rotated_prefill_output_not_rotated_back": (
        "if (rotate) oracle_hadamard_f64(out + (int64_t)p * D, D);", "(void)rotate;"),
    "e5m2_exponent_bias": ("mag = ldexp(1.0 + (double)M / 4.0, E - 15);",
                           "mag = ldexp(1.0 + (double)M / 4.0, E - 16);"),
    "e5m2_subnormal_step": ("mag = ldexp((double)M, -16);", "mag = ldexp((double)M, -15);"),
    "e5m2_saturates_to_infinity": ("if (a >= 57344.0) return (uint8_t)(sgn | 0x7B);",
                                   "if (a >= 57344.0) return (uint8_t)(sgn | 0x7C);"),
    "e5m2_ties_up": ("double mq = rint((ldexp(a, -e) - 1.0) * 4.0);",
                     "double mq = floor((ldexp(a, -e) - 1.0) * 4.0 + 0.5);"),
    "int8_round_half_up": ("double r = rint(y);                                       /* ties to even */",
                           "double r = floor(y + 0.5);"),
    "int8_asymmetric_clamp": ("if (r < -127.0) r = -127.0;", "if (r < -128.0) r = -128.0;"),
    "int8_cache_decoded_as_e4m3": ("return oracle_int8_decode(((const uint8_t*)cache)[idx]) * scale;",
                                   "return oracle_e4m3_decode(((const uint8_t*)cache)[idx]) * scale * 0.0 + oracle_int8_decode(((const uint8_t*)cache)[idx]);"),
}


def test_mutant_table_applies_to_current_source():
    src = open(SRC).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    import oracle
    old, new = MUTANTS[name]
    src = open(SRC).read()
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, str(mutated), "-o", str(so), "-lm"],
                          stderr=subprocess.DEVNULL)
    env = dict(os.environ, FP8KV_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"
