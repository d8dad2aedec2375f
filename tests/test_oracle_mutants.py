"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin fails for each: the pins are strong enough to catch a
dropped term, a wrong sign or index, a transposed operand, a wrong layout
rule or a wrong tie-break."""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "w4_oracle.c")

# (name, text to find, replacement, which occurrence (0-based) or None for all)
MUTANTS = [
    ("zero_point_7", "(double)q[row * k + kk] - 8.0", "(double)q[row * k + kk] - 7.0", None),
    ("packed_zero_point_7", "(double)qv - 8.0", "(double)qv - 7.0", None),
    ("slot_map_swapped", "(e % 2 == 0) ? e / 2 : 4 + e / 2", "(e % 2 == 0) ? 4 + e / 2 : e / 2", None),
    ("tile_row_reversed", "*r = (int)(row % 4);\n    }\n}", "*r = (int)(3 - row % 4);\n    }\n}", None),
    ("up_row_slot", "*r = (int)((row - half) % 4);", "*r = (int)(row % 4);", None),
    ("up_tile_base", "*tile = per_half + (row - half) / 4;", "*tile = (row - half) / 4;", None),
    ("group_index_dropped", "s[row * ngroups + kk / group]", "s[row * ngroups]", None),
    ("group_index_off_by_one", "s[row * ngroups + kk / group]", "s[row * ngroups + (kk + 1) % k / group]", None),
    ("q_transposed", "q[row * k + kk]", "q[kk * n + row]", None),
    ("x_reversed", "oracle_half_to_double(x[kk])", "oracle_half_to_double(x[k - 1 - kk])", None),
    ("x_dropped", "double p = w * oracle_half_to_double(x[kk]);", "double p = w;", None),
    ("abs_dropped", "mag += fabs(p);", "mag += p;", None),
    ("half_exponent_bias", "expo - 25", "expo - 24", None),
    ("half_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)", None),
    ("half_sign_dropped", "return sign ? -v : v;", "return v;", None),
    ("half_implicit_bit", "(double)(1024 + frac)", "(double)(frac)", None),
    ("silu_sign", "t / (1.0 + exp(-t))", "t / (1.0 + exp(t))", None),
    ("silu_gate_order", "oracle_silu(y[j]) * y[half + j]", "oracle_silu(y[half + j]) * y[j]", None),
    ("argmax_last_tie", "y[i] > y[best]", "y[i] >= y[best]", None),
    ("pack_pad_zero", "memset(pw, 0x88", "memset(pw, 0x00", None),
    ("pack_word_slot", "(t * nblocks + j) * 16 + 4 * r;\n            dst[0]",
     "(t * nblocks + j) * 16 + 4 * (3 - r);\n            dst[0]", None),
    ("pack_scale_slot", "(t * ngroups + g) * 8 + 2 * r;\n            dst[0]",
     "(t * ngroups + g) * 8 + 2 * (3 - r);\n            dst[0]", None),
    ("pack_byte_order", "dst[0] = (uint8_t)(word & 0xff);", "dst[0] = (uint8_t)((word >> 24) & 0xff);", None),
    ("unpack_nibble_shift", "q[row * k + 8 * j + e] = (uint8_t)((word >> (4 * slot_of_offset(e))) & 0xfu);",
     "q[row * k + 8 * j + e] = (uint8_t)((word >> (4 * e)) & 0xfu);", None),
    ("sizes_scale_bytes", "(k / group) * 8;", "(k / group) * 16;", None),
    ("gemm_x_row_fixed", "oracle_gemv_rows(q, s, xm + m * k,", "oracle_gemv_rows(q, s, xm,", None),
    ("gemm_packed_token_index", "int64_t m = mrows[i];", "int64_t m = i;", None),
    ("attn_group_map", "int32_t g = h / group;", "int32_t g = h % n_kv;", None),
    ("attn_no_max", "double w = exp(sdot * scale - mx);", "double w = exp(sdot * scale);", None),
    ("attn_page_table_ignored", "(int64_t)page_table[t / page] * n_kv", "(int64_t)(t / page) * n_kv", None),
    ("attn_scale_dropped", "            sdot *= scale;\n", "\n", None),
    ("attn_abs_dropped", "a[(int64_t)h * dim + d] += w * fabs(v);", "a[(int64_t)h * dim + d] += w * v;", None),
    ("rmsnorm_no_mean", "double r = 1.0 / sqrt(ss / (double)n + eps);", "double r = 1.0 / sqrt(ss + eps);", None),
    ("rmsnorm_gamma_dropped", "out[i] = h[i] * r * oracle_half_to_double(gamma[i]);", "out[i] = h[i] * r;", None),
    ("rmsnorm_given_no_mean", "double r = 1.0 / sqrt(sumsq / (double)n + eps);", "double r = 1.0 / sqrt(sumsq + eps);",
     None),
    ("sumsq_blocks_overlap", "i < n && i < (u + 1) * rows;", "i < n && i <= (u + 1) * rows;", None),
    ("sumsq_blocks_not_squared", "t += h[i] * h[i];", "t += h[i];", None),
    ("rope_sign", "out[i] = x[i] * c - x[i + half] * sn;", "out[i] = x[i] * c + x[i + half] * sn;", None),
    ("rope_freq", "pow(theta, -2.0 * (double)i / (double)dim)", "pow(theta, -(double)i / (double)dim)", None),
    ("act8_truncate", "float r = rintf(prod);", "float r = truncf(prod);", None),
    ("act8_fixed_inverse", "(float)oracle_half_to_double(x[kk]) * inv;", "(float)oracle_half_to_double(x[kk]) * 127.0f;", None),
    ("act8_signed_max", "float v = (float)fabs(oracle_half_to_double(x[kk]));", "float v = (float)oracle_half_to_double(x[kk]);", None),
    ("act8_scale_inverted", "volatile float sg = amax / 127.0f;", "volatile float sg = 127.0f / amax;", None),
    ("act8_block_order_identity", "{0, 4, 1, 5, 2, 6, 3, 7}", "{0, 1, 2, 3, 4, 5, 6, 7}", None),
    ("a8_act_scale_dropped", "double p = w * ((double)codes[kk] * (double)act_scales[kk / group]);",
     "double p = w * (double)codes[kk];", None),
    ("a8_packed_act_group", "((double)codes[kk] * (double)act_scales[kk / group]);\n            acc",
     "((double)codes[kk] * (double)act_scales[0]);\n            acc", None),
    ("gemm_packed_x_row_fixed", "oracle_gemv_packed_rows(pw, ps, xm + m * k,", "oracle_gemv_packed_rows(pw, ps, xm,", None),
]


def _mutate(text, find, repl, occ):
    assert find in text, f"mutation anchor not found: {find!r}"
    if occ is None:
        return text.replace(find, repl)
    idx = -1
    for _ in range(occ + 1):
        idx = text.index(find, idx + 1)
    return text[:idx] + repl + text[idx + len(find):]


@pytest.mark.parametrize("name,find,repl,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl, occ, tmp_path):
    text = open(SRC).read()
    mutated = _mutate(text, find, repl, occ)
    assert mutated != text
    src = tmp_path / f"{name}.c"
    src.write_text(mutated)
    lib = oracle.build(str(src), str(tmp_path / f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except ValueError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
