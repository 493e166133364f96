"""Planted-mistake check for the oracle's pins (CPU only).

Each mutant is the oracle's C source with one plausible mistake (a wrong
sign, a dropped term, an off-by-one, a wrong head index, ...). It is compiled
to a temporary library and every pin in ``test_oracle_pins`` is run against
it; at least one pin must fail. The mistakes are planted only in throw-away
copies of the oracle, never in the product path.
"""

import math
import os

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "bsp_oracle.c")).read()

MUTANTS = {
    "gap_sign": [("gap = m[r] - mloc[r];", "gap = mloc[r] - m[r];")],
    "non_strict": [("int skip = (mingap > lam);", "int skip = (mingap >= lam);")],
    "no_acc_rescale": [("for (int d = 0; d < D; ++d) a[d] *= alpha;", "")],
    "no_l_rescale": [("l[r] = alpha * l[r] + rowsum;", "l[r] = l[r] + rowsum;")],
    "running_max_frozen": [("m[r] = mnew;", "")],
    "causal_strict": [("if (c0 + c <= qi) {", "if (c0 + c < qi || (c0 + c == 0 && qi == 0)) {")],
    "drop_diagonal_block": [("const int nblk = (off + r1 - 1) / block_k + 1;",
                             "const int nblk = (off + r1 - 1) / block_k + ((off + r1 - 1) % block_k == block_k - 1);")],
    "gqa_modulo": [("const int g = h / group;", "const int g = h % n_heads_kv;")],
    "scale_wrong": [("const double scale = 1.0 / sqrt((double)head_dim);",
                     "const double scale = 1.0 / (double)head_dim;")],
    "lse_log2": [("lse_w[r] = m[r] + log(l[r]);", "lse_w[r] = m[r] + log2(l[r]);")],
    "any_row_rule": [("double mingap = INFINITY;", "double mingap = -INFINITY;"),
                     ("if (gap < mingap) mingap = gap;", "if (gap > mingap) mingap = gap;")],
    "masked_row_blocks": [("gap = INFINITY;             /* nothing visible in this block */",
                           "gap = -INFINITY;")],
    "k_scale_ignored": [("const double sk = k_scale ? k_scale[g] : 1.0;", "const double sk = 1.0;")],
    "v_offset": [("elem(v, ((size_t)(kbase + c0 + c) * n_heads_kv + g) * D + d, in_dtype) * sv;",
                  "elem(v, ((size_t)(kbase + c0 + (c + 1) % nc) * n_heads_kv + g) * D + d, in_dtype) * sv;")],
    "bf16_widen_shift": [("const uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;",
                          "const uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 15;")],
    "fp8_bias": [("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)")],
    "chunk_offset_dropped": [("const int off = Lk - L;", "const int off = 0 * (Lk - L);")],
    "chunk_keys_from_query_base": [("const int kbase = cu_seqlens_k ? cu_seqlens_k[s] : base;",
                                    "const int kbase = base;")],
    "chunk_blocks_end_at_query_length": [("const int c1 = (c0 + block_k < Lk) ? c0 + block_k : Lk;\n                const int nc",
                                          "const int c1 = (c0 + block_k < L) ? c0 + block_k : L;\n                const int nc")],
    "lambda_per_sequence_ignored": [("const double lam = lambda_seq ? lambda_seq[s] : lambda;",
                                     "const double lam = lambda;")],
}


def _pin_calls():
    """Every pin test as a zero-argument callable (parametrisations expanded)."""
    calls = []
    for case in pins.CASES:
        calls.append(lambda c=case: pins.test_dense_limit_equals_naive_softmax(c))
        for lam in [0.0, 2.0]:
            calls.append(lambda c=case, l=lam: pins.test_skip_set_matches_brute_force(c, l))
            calls.append(lambda c=case, l=lam: pins.test_kept_key_closed_form(c, l))
    for lam in [0.0, math.inf]:
        calls.append(lambda l=lam: pins.test_probabilities_sum_to_one_and_reproduce_output(l))
    calls += [pins.test_block_zero_never_skipped_and_output_finite,
              pins.test_golden_worked_examples,
              pins.test_tie_at_lambda_is_kept_on_random_integer_scores,
              pins.test_fp8_scales_are_applied_per_head,
              pins.test_gqa_equals_repeated_mha,
              lambda: pins.test_storage_types_widen_exactly("bf16"),
              lambda: pins.test_storage_types_widen_exactly("fp8"),
              pins.test_lambda_per_sequence_equals_separate_runs]
    for case in pins.CHUNK_CASES:
        calls.append(lambda c=case: pins.test_chunked_dense_limit_equals_naive_softmax(c))
        calls.append(lambda c=case: pins.test_chunked_skip_set_and_kept_keys_match_brute_force(c, 1.5))
    calls.append(lambda: pins.test_chunk_after_whole_tiles_equals_rows_of_full_prefill(1))
    return calls


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    src = SRC
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor for {name} not found"
        src = src.replace(old, new)
    lib = oracle.load_library(oracle.compile_source(src, str(tmp_path / f"mut_{name}.so")))
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = 0
    for call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError, FloatingPointError):
            failed += 1
            break
    assert failed > 0, f"no pin detects mutant {name}"
