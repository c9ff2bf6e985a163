"""Mutation test of the oracle's pins.

Each case plants one plausible mistake in a copy of oracle/bq_oracle.c (on the CPU, in a
temporary directory), builds it, and requires at least one pin of oracle_pins.py to fail on
it.  A mutant that every pin accepts would mean the pins cannot see that kind of mistake.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble_order_swapped": ("(uint8_t)((hi << 4) | lo)", "(uint8_t)((lo << 4) | hi)"),
    "pad_nibble_not_zero": ("codes[2 * j + 1] : 0;", "codes[2 * j + 1] : 15;"),
    "ties_to_higher_index": ("if (2.0 * (double)y > (double)c[best]",
                             "if (2.0 * (double)y >= (double)c[best]"),
    "absmax_keeps_infinities": ("if (isfinite(v) && fabsf(v) > a)", "if (!isnan(v) && fabsf(v) > a)"),
    "absmax_signed_max": ("if (isfinite(v) && fabsf(v) > a) a = fabsf(v);",
                          "if (isfinite(v) && v > a) a = v;"),
    "divide_instead_of_reciprocal": ("float y = xs * r;", "float y = xs / as;"),
    "guard_dropped": ("if (a < 0x1p-64f) return 0x1p64f;", "if (0) return 0x1p64f;"),
    "zero_code_is_index_0": ("int bqo_zero_code(const float* c, int K) { return bqo_nearest(0.0f, c, K); }",
                             "int bqo_zero_code(const float* c, int K) { (void)c; (void)K; return 0; }"),
    "narrowing_truncates": ("return rint(a / quantum) * quantum;", "return floor(a / quantum) * quantum;"),
    "f16_subnormal_scale": ("mag = ldexpf((float)m, -24);", "mag = ldexpf((float)m, -25);"),
    "bf16_exponent_bias": ("mag = ldexpf((float)(128 + m), e - 134);", "mag = ldexpf((float)(128 + m), e - 133);"),
    "sequential_sum": ("return pairwise_sum(a, n, 0, len);",
                       "double S = 0; for (int64_t i = 0; i < n; ++i) S += a[i]; return S;"),
    "mean_in_binary32": ("return (float)(S / (double)nb);", "return (float)S / (float)nb;"),
    "mean_not_subtracted": ("d[b - b_lo] = absmax[b] - mean;", "d[b - b_lo] = absmax[b];"),
    "table_negative_zero_kept": ("if (v == 0.0f) v = 0.0f; /* -0.0 -> +0.0 */", ""),
    "table_range_unchecked": ("if (!isfinite(v) || v < -1.0f || v > 1.0f) return -1;", ""),
    "table_order_unchecked": ("if (k > 0 && !(v > c_out[k - 1])) return -1;", ""),
    "mean_not_added_back": ("a[b] = scaled + mean;", "a[b] = scaled;"),
    "q32_nibbles_swapped": ("int lo = blk[2 + j] & 0x0f, hi = blk[2 + j] >> 4;",
                            "int hi = blk[2 + j] & 0x0f, lo = blk[2 + j] >> 4;"),
    "q32_offset_7": ("(float)(lo - 8) * d", "(float)(lo - 7) * d"),
    "q8_unsigned_codes": ("int q = (int8_t)blk[2 + j];", "int q = (uint8_t)blk[2 + j];"),
    "dequant_wrong_block": ("* absmax[i / B];", "* absmax[(i + 1) / B];"),
    "linear_transposed_weight": ("const int64_t flat = n * K + k;", "const int64_t flat = k * N + n;"),
    "linear_wrong_block": ("const float scale = absmax[flat / B];", "const float scale = absmax[flat / B / 2];"),
    "linear_drops_last_term": ("s += (double)load_elem(x, dtype, m * K + k) * (double)w;",
                               "if (k + 1 < K) s += (double)load_elem(x, dtype, m * K + k) * (double)w;"),
    "linear_binary32_sum": ("      double s = 0.0;\n      for (int64_t k = 0; k < K; ++k) {\n        const int64_t flat",
                            "      float s = 0.0f;\n      for (int64_t k = 0; k < K; ++k) {\n        const int64_t flat"),
    "gemm_weight_not_rounded": ("""        const float w16 = dtype == BQO_F16 ? bqo_f16_to_f32(bqo_f32_to_f16(w32))
                                           : bqo_bf16_to_f32(bqo_f32_to_bf16(w32));""",
                                "        const float w16 = w32;"),
    "gemm_rounds_to_the_other_type": ("const float w16 = dtype == BQO_F16 ?", "const float w16 = dtype != BQO_F16 ?"),
    "gemm_transposed_weight": ("const int64_t f = n * K + k;", "const int64_t f = k * N + n;"),
    "gemm_binary32_sum": ("double acc = 0.0;", "float acc = 0.0f;"),
    "iq_flip_strongest": ("      if (p < w) {", "      if (p > w) {"),
    "iq_no_parity_correction": ("    dot = fmaf(-2.0f, w, dot);\n", ""),
    "iq_scale_ties_to_higher": ("if (l == 0 || sum < best_sum)", "if (l == 0 || sum <= best_sum)"),
    "iq_entry_ties_to_higher": ("iq_entry_qnorm(q), s);\n    if (e == 0 || err < best)",
                                "iq_entry_qnorm(q), s);\n    if (e == 0 || err <= best)"),
    "iq_sign_bits_at_8": ("(uint16_t)(e | ((signs & 0x7f) << 9))", "(uint16_t)(e | ((signs & 0x7f) << 8))"),
    "iq_scale_nibbles_swapped": ("(uint8_t)(ls[2 * i] | (ls[2 * i + 1] << 4))", "(uint8_t)(ls[2 * i + 1] | (ls[2 * i] << 4))"),
    "iq_local_scale_even": ("float s = d * (float)(2 * l + 1) * 0.125f; /* I4 */", "float s = d * (float)(2 * l + 2) * 0.125f; /* I4 */"),
    "iq_decode_quarter": ("float dl = d * (float)(2 * ls + 1) * 0.125f;", "float dl = d * (float)(2 * ls + 1) * 0.25f;"),
    "iq_decode_parity_dropped": ("      signs |= parity << 7;\n", ""),
    "iq_nonfinite_kept": ("float t = isfinite(x[j]) ? x[j] : 0.0f; /* I1 */", "float t = x[j];"),
    "iq_negative_scale_accepted": ("if ((d_bits & 0x7c00) == 0x7c00 || (d_bits & 0x8000)) return 1;",
                                   "if ((d_bits & 0x7c00) == 0x7c00) return 1;"),
    "iq_negative_zero_rejected": ("if ((d_bits & 0x7fff) == 0) return 0;", "if (d_bits == 0) return 0;"),
    "iq_group_of_one_vector": ("+ iq_best_entry(&vec[2 * g + 1], grid, s, &e1);", "; (void)e1;"),
    "iq_error_sign_flipped": ("fmaf(-2.0f * s, dot, xn)", "fmaf(2.0f * s, dot, xn)"),
    "iq1_scale_order": ("float d = (amax / 16.875f) * 0.61f;", "float d = (amax * 0.61f) / 16.875f;"),
    "iq1_scale_not_saturated": ("if ((h & 0x7c00) == 0x7c00) h = 0x7bff;", ""),
    "iq1_choice_ties_to_higher": ("if (c == 0 || sum < best_sum)", "if (c == 0 || sum <= best_sum)"),
    "iq1_entry_ties_to_higher": ("float err = iq1_error(xn, dot, xsum, qn, qs, dl, delta);\n    if (e == 0 || err < best)",
                                 "float err = iq1_error(xn, dot, xsum, qn, qs, dl, delta);\n    if (e == 0 || err <= best)"),
    "iq1_delta_sign_inverted": ("float sdot = fmaf(delta, xsum, dot);", "float sdot = fmaf(-delta, xsum, dot);"),
    "iq1_no_delta_square_term": ("float snorm = qn + 2.0f * delta * qs + 8.0f * delta * delta;",
                                 "float snorm = qn + 2.0f * delta * qs;"),
    "iq1_first_vector_only": ("sum += iq1_best_entry(", "if (l == 0) sum += iq1_best_entry("),
    "iq1_high_bits_shifted": ("qh |= (uint32_t)(e >> 8) << (3 * l);", "qh |= (uint32_t)(e >> 8) << (3 * l + 1);"),
    "iq1_scale_bits_at_11": ("uint32_t qh = (uint32_t)(best_c & 7) << 12", "uint32_t qh = (uint32_t)(best_c & 7) << 11"),
    "iq1_nonfinite_kept": ("x[i] = isfinite(x_in[i]) ? x_in[i] : 0.0f; /* J1 */", "x[i] = x_in[i];"),
    "iq1_decode_delta_inverted": ("const float delta = (qh & 0x8000) ? -0.125f : 0.125f;",
                                  "const float delta = (qh & 0x8000) ? 0.125f : -0.125f;"),
    "iq1_decode_even_scale": ("const float dl = d * (float)(2 * ((qh >> 12) & 7) + 1);",
                              "const float dl = d * (float)(2 * ((qh >> 12) & 7) + 2);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation target not found (or not unique): %r" % old
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(path, os.path.join(tmp_path, "libmutant.so")))
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception:  # any rejection counts
            caught.append(pin.__name__)
            break
    assert caught, "no pin detects the planted mistake %s" % name
