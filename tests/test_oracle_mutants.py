"""Plant plausible mistakes in copies of oracle.c; every one must fail a pin.

This shows the pins are discriminating: a dropped term, a wrong sign, a wrong
index, a transposed operand or a flipped tie-break anywhere in the oracle is
caught by at least one check against the mathematics.  Mutants are built in a
temporary directory on the CPU; the real oracle is untouched.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("tie_to_higher_index", "return a < b;", "return a > b;"),
    ("tie_not_strict", "if (ka > kb) return 1;", "if (ka >= kb) return 1;"),
    ("dot_drops_last_term", "for (int64_t i = 0; i < H; ++i) {", "for (int64_t i = 0; i + 1 < H; ++i) {"),
    ("dot_transposed_operand", "const uint16_t* wr = w + e * H;", "const uint16_t* wr = w + (e % (M > 0 ? M : 1)) * H;"),
    ("dot_wrong_x_row", "const uint16_t* xr = x + t * H;", "const uint16_t* xr = x;"),
    ("absdot_signed", "mag += fabs(p);", "mag += p;"),
    ("softplus_drops_linear_term", "double softplus = fmax(v, 0.0) + log1p(exp(-fabs(v)));",
     "double softplus = log1p(exp(-fabs(v)));"),
    ("softplus_sign_flip", "double softplus = fmax(v, 0.0) + log1p(exp(-fabs(v)));",
     "double softplus = fmax(v, 0.0) + log1p(exp(fabs(v)));"),
    ("softplus_no_sqrt", "score[e] = sqrt(softplus);", "score[e] = softplus;"),
    ("softmax_no_normalise", "for (int64_t e = 0; e < E; ++e) score[e] = unbiased[e] / Z;",
     "for (int64_t e = 0; e < E; ++e) score[e] = unbiased[e];"),
    ("softmax_wrong_shift_sign", "unbiased[e] = exp((double)l[e] - m);", "unbiased[e] = exp(m - (double)l[e]);"),
    ("key_ignores_bias", "kv = s32 + bias[e];", "kv = s32;"),
    ("key_bias_on_logit", "kv = s32 + bias[e];", "kv = l[e] + bias[e];"),
    ("key_is_score_without_bias", "kv = l[e];", "kv = (float)score[e] + 0.0f * l[e];"),
    ("weights_use_key", "wgt = unb[e] / total;", "wgt = key[e] / total;"),
    ("renorm_over_all_experts", "for (int j = 0; j < k; ++j) total += unb[top_idx[j]];",
     "for (int j = 0; j < E; ++j) total += unb[j];"),
    ("no_renorm_uses_unnormalised", "wgt = score[e];", "wgt = unb[e];"),
    ("insertion_skips_top_slot", "while (pos > 0 && precedes(", "while (pos > 1 && precedes("),
    ("insertion_ignores_full_list", "if (filled == k && !precedes(", "if (filled == k && precedes("),
    ("table_token_from_rank", "int token = s / k;", "int token = s % 2;"),
    ("table_tail_zero", "ids[i] = -1;", "ids[i] = 0;"),
    ("table_mask_overwrite", "token_mask[pos] |= 1 << token;", "token_mask[pos] = 1 << token;"),
    ("table_slot_map_raw", "slot_to_unique[s] = pos;", "slot_to_unique[s] = s;"),
    ("mx_nibble_order", "int code = (col % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "int code = (col % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    ("mx_scale_bias", "ldexp(oracle_e2m1_value(code), sc - 127)", "ldexp(oracle_e2m1_value(code), sc - 128)"),
    ("e2m1_subnormal_half", "? 0.5 * man", "? 0.25 * man"),
    ("e2m1_exponent_bias", "ldexp(1.0 + 0.5 * man, ex - 1)", "ldexp(1.0 + 0.5 * man, ex)"),
    ("table_pair_width_only", "int n = M * k;", "int n = (M > 2 ? 2 : M) * k;"),
    ("table_mask_two_tokens", "token_mask[pos] |= 1 << token;", "token_mask[pos] |= 1 << (token & 1);"),
    ("bf16_ties_away", "mag = (lo & 1u) ? hi : lo;  /* tie: the even neighbour */", "mag = hi;"),
    ("bf16_truncates", "if (a - vlo < vhi - a)", "if (1)"),
    ("gather_no_intermediate_round", "const float routed = bf16_to_float(oracle_bf16_round(acc));",
     "const float routed = acc;"),
    ("gather_reversed_slots", "for (int j = 0; j < k; ++j) {\n                int64_t r = slot_rows[t * k + j];",
     "for (int j = k - 1; j >= 0; --j) {\n                int64_t r = slot_rows[t * k + j];"),
    ("gather_fused_multiply_add",
     "const float p = weights[t * k + j] * bf16_to_float(y[r * D + d]);\n                acc = acc + p;",
     "acc = fmaf(weights[t * k + j], bf16_to_float(y[r * D + d]), acc);"),
    ("gather_double_accumulator", "float acc = 0.0f;", "double acc = 0.0;"),
    ("gather_remote_reads_row0", "if (r < 0) continue;", "if (r < 0) r = 0;"),
    ("gather_drops_shared", "const float sum = routed + bf16_to_float(shared[t * D + d]);",
     "const float sum = routed;"),
    ("table_rows_token_inclusive", "for (int q = 0; q < t; ++q) within", "for (int q = 0; q <= t; ++q) within"),
    ("table_rows_no_block_offset", "for (int v = 0; v < u; ++v)", "for (int v = 0; v < 0; ++v)"),
    ("gemm1_expert_by_slot", "const uint16_t* wexp = w1 + id * F * D;",
     "const uint16_t* wexp = w1 + (int64_t)(u % E) * F * D;"),
    ("gemm1_transposed_weights", "const double prod = bf16_value(xr[d]) * bf16_value(wrow[d]);",
     "const double prod = bf16_value(xr[d]) * bf16_value(wexp[((d * F + f) % (F * D))]);"),
    ("gemm1_tokens_reversed", "const uint16_t* xr = x + (int64_t)t * D;",
     "const uint16_t* xr = x + (int64_t)(M - 1 - t) * D;"),
    ("gemm1_drops_last_term", "for (int64_t d = 0; d < D; ++d) {\n                    const double prod",
     "for (int64_t d = 0; d + 1 < D; ++d) {\n                    const double prod"),
    ("gemm1_absdot_signed", "amag += fabs(prod);", "amag += prod;"),
    ("e4m3_exponent_bias", "ldexp(1.0 + frac / 8.0, biased - 7)", "ldexp(1.0 + frac / 8.0, biased - 8)"),
    ("e4m3_subnormal_exponent", "ldexp(frac / 8.0, -6)", "ldexp(frac / 8.0, -7)"),
    ("e4m3_nan_pattern", "if (biased == 15 && frac == 7) return NAN;", "if (biased == 15 && frac >= 6) return NAN;"),
    ("e4m3_sign_dropped", "return negative ? -magnitude : magnitude;", "return magnitude;"),
    ("mx8_scale_bias", "w[row * H + idx] = ldexp(v, s8 - 127);", "w[row * H + idx] = ldexp(v, s8 - 126);"),
]


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, src_text, name, old, new):
    assert src_text.count(old) == 1, f"mutation anchor not unique/absent: {old!r}"
    mutated = src_text.replace(old, new)
    path = tmp_path / "oracle_mut.c"
    path.write_text(mutated)
    lib = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(lib, sources=[str(path)], extra_flags=["-w"])
    orc = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, OverflowError) as exc:
            failures.append((pin.__name__, type(exc).__name__))
    assert failures, f"planted mistake {name} passed every pin"
