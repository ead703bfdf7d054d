"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (on the CPU, in a
temporary directory), builds it, swaps it in for the real oracle and runs the pin
tests of test_oracle.py: at least one pin must fail.  The real oracle is restored
afterwards.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("nibble_order_high_first", "word |= (uint32_t)(codes[(size_t)n * K + 8 * w + j] & 15u) << (4 * j);",
     "word |= (uint32_t)(codes[(size_t)n * K + 8 * w + j] & 15u) << (28 - 4 * j);"),
    ("unpack_reads_high_first", "return (int)((qweight[(size_t)n * (K / 8) + k / 8] >> (4 * (k % 8))) & 15u);",
     "return (int)((qweight[(size_t)n * (K / 8) + k / 8] >> (28 - 4 * (k % 8))) & 15u);"),
    ("zero_dropped", "w[k] = (double)(q - z) * s;", "w[k] = (double)(q) * s;"),
    ("sign_flipped", "w[k] = (double)(q - z) * s;", "w[k] = (double)(z - q) * s;"),
    ("scale_dropped", "w[k] = (double)(q - z) * s;", "w[k] = (double)(q - z);"),
    ("group_of_64", "int g = k / group;\n        int q = q_at", "int g = k / 64 % (K / group);\n        int q = q_at"),
    ("zero_row_index", "return (int)((qzeros[(size_t)(n / 8) * G + g] >> (4 * (n % 8))) & 15u);",
     "return (int)((qzeros[(size_t)(n % 8) * G + g] >> (4 * (n / 8 % 8))) & 15u);"),
    ("scale_transposed", "double s = oracle_f16_to_f64(scales[(size_t)n * G + g]);",
     "double s = oracle_f16_to_f64(scales[(size_t)g * N_unused + n]);"),
    ("x_row_stride", "acc += oracle_bf16_to_f64(X[(size_t)m * K + k]) * w[k];",
     "acc += oracle_bf16_to_f64(X[(size_t)m * 8 + k]) * w[k];"),
    ("argmax_ties_high", "if (row[n] > row[best])", "if (row[n] >= row[best])"),
    ("accept_counts_all_matches", "while (L < M && argmax[L] == draft[L])\n        ++L;",
     "for (int i = 0; i < M; ++i)\n        L += argmax[i] == draft[i];"),
    ("f16_bias_off_by_one", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    ("bf16_low_half", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h;"),
    ("gidx_ignored", "int g = g_idx[k];", "int g = k / group;"),
    ("gidx_zero_from_k", "w[k] = (double)(q_at(qweight, K, n, k) - z_at(qzeros, G, n, g)) *\n                       oracle_f16_to_f64(scales[(size_t)n * G + g]);",
     "w[k] = (double)(q_at(qweight, K, n, k) - z_at(qzeros, G, n, k / group)) *\n                       oracle_f16_to_f64(scales[(size_t)n * G + g]);"),
    ("swa_unscaled", "double scale = 1.0 / sqrt((double)D);", "double scale = 1.0;"),
    ("swa_window_off_by_one", "int j0 = p - window + 1 > 0 ? p - window + 1 : 0;", "int j0 = p - window > 0 ? p - window : 0;"),
    ("swa_kv_head_modulo", "int kv = h / grp;", "int kv = h % Hkv;"),
    ("swa_block_causal_in_block", "int j1 = T;      /* one past the last key seen: the whole block */",
     "int j1 = p + 1;"),
    ("swa_block_window_from_block_start", "int c0 = p - window + 1 > 0 ? p - window + 1 : 0; /* first context key in the window */",
     "int c0 = b0 - window + 1 > 0 ? b0 - window + 1 : 0;"),
    ("swa_v_untransposed", "acc += sc[j - j0] * oracle_bf16_to_f64(Vt[((size_t)kv * D + d) * T + j]);",
     "acc += sc[j - j0] * oracle_bf16_to_f64(Vt[((size_t)j * Hkv + kv) * D + d]);"),
    ("quantize_ties_away", "if (d > 0.0 || (d == 0.0 && fmod(r, 2.0) != 0.0))", "if (d >= 0.0)"),
    ("quantize_round_after_zero", "q = round_quotient(w, s) + z;", "q = round_quotient(w + z * s, s);"),
    ("quantize_truncates", "if (d > 0.0 || (d == 0.0 && fmod(r, 2.0) != 0.0))\n        r += 1.0;",
     "if (0)\n        r += 1.0;"),
    ("quantize_no_low_clamp", "if (q < 0.0)\n                q = 0.0;", "if (q < -100.0)\n                q = 0.0;"),
    ("quantize_group_of_64", "int g = k / group;\n            double w = oracle_bf16_to_f64(W",
     "int g = k / 64 % G;\n            double w = oracle_bf16_to_f64(W"),
    ("silu_sign_of_exponent", "Y[i] = G[i] / (1.0 + exp(-G[i])) * U[i];", "Y[i] = G[i] / (1.0 + exp(G[i])) * U[i];"),
    ("silu_without_gate_factor", "Y[i] = G[i] / (1.0 + exp(-G[i])) * U[i];", "Y[i] = 1.0 / (1.0 + exp(-G[i])) * U[i];"),
    ("gated_up_dropped", "Y[i] = G[i] / (1.0 + exp(-G[i])) * U[i];", "Y[i] = G[i] / (1.0 + exp(-G[i]));"),
]

PIN_TESTS = [
    lambda: pins.test_bf16_decode_textbook_values(),
    lambda: pins.test_f16_decode_textbook_values(),
    lambda: pins.test_pack_layout_golden(),
    lambda: pins.test_linear_worked_by_hand(),
    lambda: pins.test_onehot_picks_one_weight(),
    lambda: pins.test_equal_codes_closed_form(),
    lambda: pins.test_dyadic_inputs_exact(),
    lambda: pins.test_verify_golden_cases(),
    lambda: pins.test_gidx_sequential_is_the_plain_oracle(),
    lambda: pins.test_gidx_onehot_picks_its_group(),
    lambda: pins.test_gidx_column_permutation_invariance(),
    lambda: pins.test_swa_window_of_one_returns_own_value(),
    lambda: pins.test_swa_equal_keys_give_the_window_mean(),
    lambda: pins.test_swa_matches_masked_softmax_formulation(5),
    lambda: pins.test_swa_block_single_query_is_causal(),
    lambda: pins.test_swa_block_equal_keys_give_the_mean_over_context_window_and_block(),
    lambda: pins.test_swa_block_is_invariant_to_permuting_the_block(),
    lambda: pins.test_swa_block_matches_masked_softmax_formulation(3),
    lambda: pins.test_quantize_worked_by_hand(),
    lambda: pins.test_quantize_returns_on_grid_weights_to_their_codes(0),
    lambda: pins.test_quantize_matches_exact_rational_rounding(),
    lambda: pins.test_silu_closed_forms(),
    lambda: pins.test_silu_odd_part_identity(),
    lambda: pins.test_gated_applies_silu_to_the_gate_and_scales_by_up(),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, mut, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert orig in src, "mutation anchor not found: " + name
    mutated = src.replace(orig, mut, 1)
    if "N_unused" in mutated:
        mutated = mutated.replace("static void dequant_row(", "static const int N_unused = 8;\nstatic void dequant_row(", 1)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off",
                           "-o", str(so), str(path), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle._bind(str(so)))
    failed = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, Exception):
            failed += 1
    assert failed > 0, "no pin caught mutant " + name
