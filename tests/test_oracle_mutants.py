"""Planted mistakes in the oracle's hot-path functions, each caught by a pin.

Every mutant is one plausible slip (a wrong index, a flipped sign, a dropped
term, an off-by-one boundary, a transposed operand, a different rounding
rule) planted in a copy of the oracle built in a temporary directory.  The
test runs the named pins, whose references come from closed forms, hand-
worked cases or brute force, against the mutant and requires each of them to
fail.  None of these mutants moves an access out of bounds."""

import pytest

import test_oracle_backward as bwd
import test_oracle_formats as fmt
import test_oracle_lse as lse
import test_oracle_relayout as rel
from oracle_mutant import build_oracle_mutant

MUTANTS = {
    # seq->head reads the next rank's head block
    "relayout_head_block": (
        "int64_t i = (((j * B + b) * Sp + s) * H + r * Hp + h) * D;",
        "int64_t i = (((j * B + b) * Sp + s) * H + ((r + 1) % P) * Hp + h) * D;",
        [(rel.test_dense_matches_global_closed_form, dict(shape=(2, 3, 8, 4, 8))),
         (rel.test_dense_golden_hand_case, {})]),
    # the varlen pieces rounded up instead of down
    "piece_bounds_ceil": (
        "static int64_t piece_start(int64_t p, int64_t L, int64_t P) { return (p * L) / P; }",
        "static int64_t piece_start(int64_t p, int64_t L, int64_t P) { return (p * L + P - 1) / P; }",
        [(rel.test_varlen_plan_by_counting, dict(case=([17, 33, 2, 64], 4, 3, 8, 4)))]),
    # LSE = max - log(sum)
    "lse_sign": (
        "return (double)m + log((double)s);",
        "return (double)m - log((double)s);",
        [(lse.test_lse_golden_cases, {})]),
    # the sum's sign not checked (a zero sum would still give -inf through
    # log(0), so the planted slip admits negative sums)
    "lse_negative_sum_valid": (
        "if (isfinite(m) && isfinite(s) && s > 0.0f)",
        "if (isfinite(m) && isfinite(s))",
        [(lse.test_lse_golden_cases, {})]),
    # combine weights exp(M - L) instead of exp(L - M)
    "combine_weight_sign": (
        "        double w = exp(part_l[p] - M);\n        Z += w;",
        "        double w = exp(M - part_l[p]);\n        Z += w;",
        [(lse.test_combine_golden_cases, {})]),
    # the combined LSE without the max
    "combine_lse_drops_max": (
        "*lse_out = M + log(Z);",
        "*lse_out = log(Z);",
        [(lse.test_combine_golden_cases, {})]),
    # causal rule: a piece starting at the token itself taken as masked
    "causal_strict": (
        "return a < e && a <= k;",
        "return a < e && a < k;",
        [(lse.test_causal_varlen_attention_equals_masked_combine, dict(lengths=[9, 1, 16], P=4))]),
    # causal rule: empty pieces taken as valid
    "causal_empty_piece_valid": (
        "return a < e && a <= k;",
        "return a <= k;",
        [(lse.test_causal_varlen_attention_equals_masked_combine, dict(lengths=[5, 12], P=8))]),
    # gradient of the LSEs without the upstream LSE gradient
    "grad_drops_g_lse": (
        "d_l[p] = w * (gp - g_out + g_lse);",
        "d_l[p] = w * (gp - g_out);",
        [(bwd.test_golden_closed_forms, {}),
         (bwd.test_finite_differences_of_forward, dict(P=5, D=7, n_invalid=2, g_lse=-1.3))]),
    # gradient of the LSEs with the mean term's sign flipped
    "grad_sign": (
        "d_l[p] = w * (gp - g_out + g_lse);",
        "d_l[p] = w * (gp + g_out + g_lse);",
        [(bwd.test_golden_closed_forms, {}),
         (bwd.test_finite_differences_of_forward, dict(P=2, D=5, n_invalid=0, g_lse=0.0))]),
    # bf16/fp16 rounding with ties away from zero instead of to even
    "rounding_ties_away": (
        "double q = nearbyint(x / spacing);",
        "double q = round(x / spacing);",
        [(fmt.test_bf16_round_brute_force_ties_and_double_precision, {})]),
    # pack chunks laid out [P_dst][P_src] instead of [P_src][P_dst]
    "pack_chunks_transposed": (
        "char* obase = dst + (p * P + r) * chunk;",
        "char* obase = dst + (r * P + p) * chunk;",
        [(lse.test_pack_matches_slicing_and_legacy_path, dict(scatter_dim=1, P=2, T=4, H=4, Dv=8))]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_oracle_mistakes(orc, tmp_path, name):
    old, new, pins = MUTANTS[name]
    mutant = build_oracle_mutant(orc, tmp_path, old, new, name)
    for pin, kwargs in pins:
        pin(orc, **kwargs)               # the pin holds for the oracle itself
        with pytest.raises(AssertionError):
            pin(mutant, **kwargs)        # and fails for the mutant
