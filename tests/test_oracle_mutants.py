"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them: a dropped term, a wrong sign, index or
comparison, a transposed operand.  Each mutant is oracle.c with one textual
edit, built with gcc into a temporary library and swapped in for the real
oracle while a chosen set of pin tests runs against it."""
import os
import subprocess
import tempfile

import pytest

import oracle
from . import test_oracle_attention as TA
from . import test_oracle_sampler as TS
from . import test_oracle_kvcache as TK
from . import test_oracle_temperature as TT
from . import test_oracle_topp as TP
from . import test_oracle_tree as TR
from . import test_oracle_typical as TY
from . import test_oracle_tree_commit as TC

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# Ordered so that pins whose inputs leave slack in the block table run first: a
# mutant that reads one position too far then hits a poisoned slot, not memory
# past the end of the table.
ATTN_PINS = [
    TA.test_causal_mask_offset, TA.test_gqa_head_map_uses_floor_h_over_G,
    TA.test_two_visible_keys_closed_form, TA.test_zero_query_gives_mean_of_visible_values,
    TA.test_bf16_decoder_exhaustive, TA.test_e4m3_decoder_exhaustive,
] + [lambda c=c: TA.test_oracle_matches_library_attention(*c) for c in TA.CASES]
SAMPLE_PINS = [
    lambda: TS.test_every_emitted_position_follows_target("noisy"),
    TS.test_boundary_uniforms, TS.test_two_token_worked_example,
    TS.test_residual_mass_identity_on_config_rows, TS.test_accept_ratio_matches_library_softmax,
    TS.test_draft_equal_to_target_accepts_all_and_draws_bonus,
    lambda: TS.test_mean_tokens_per_round_closed_form(4, 0.6),
]

KV_PINS = [
    TK.test_bf16_encoder_matches_library_cast, TK.test_e4m3_encoder_matches_library_cast_within_range,
    TK.test_e4m3_encoder_round_trips_every_finite_code_and_saturates, TK.test_e4m3_encoder_divides_by_the_scale_in_float,
    lambda: TK.test_append_writes_exactly_the_new_positions("f32"),
    lambda: TK.test_append_writes_exactly_the_new_positions("bf16"),
    lambda: TK.test_append_writes_exactly_the_new_positions("fp8"),
    TK.test_append_then_attention_equals_attention_on_the_full_cache,
    TK.test_rollback_keeps_the_loop_invariant, TK.test_rollback_extremes,
]

TEMP_PINS = [
    TT.test_target_row_matches_library_softmax, TT.test_greedy_limit_is_greedy_decoding,
    TT.test_temperature_rescales_the_logits, lambda: TT.test_every_emitted_position_follows_tempered_target(0.5, 0.5),
]

TOPP_PINS = [
    TP.test_cut_matches_the_ascending_cumsum_recipe, TP.test_cut_matches_the_threshold_form_with_ties,
    TP.test_vanishing_top_p_is_the_greedy_limit, TP.test_full_or_nan_top_p_changes_nothing,
]

TREE_PINS = [
    TR.test_chain_masks_are_the_causal_mask, lambda: TR.test_node_sees_exactly_prefix_and_root_path("binary3"),
    TR.test_chain_tree_is_the_chain_sampler, TR.test_third_sibling_ratio_worked_example,
    lambda: TR.test_exact_law_of_recursive_rejection(3),
]

TYPICAL_PINS = [
    TY.test_entropy_matches_library_and_closed_forms, TY.test_uniform_target_closed_form,
    TY.test_one_hot_target_accepts_exactly_its_argmax, TY.test_zero_eps_accepts_every_positive_draft,
    TY.test_two_token_worked_example, TY.test_token_after_the_prefix_follows_its_row,
]

COMMIT_PINS = [
    TC.test_chain_path_moves_nothing_and_is_the_rollback,
    lambda: TC.test_committed_cache_is_prefix_root_and_path("bf16"),
    lambda: TC.test_committed_cache_is_prefix_root_and_path("fp8"),
    TC.test_attention_after_commit_sees_the_linear_sequence,
]

# (name, original text, replacement, pins expected to catch it)
MUTANTS = [
    ("head map h % Hkv", "const int g = h / G;", "const int g = h % Hkv;", ATTN_PINS),
    ("causal offset one short", "const int64_t n_vis = L - T + 1 + t;", "const int64_t n_vis = L - T + t;", ATTN_PINS),
    ("causal offset one long", "const int64_t n_vis = L - T + 1 + t;", "const int64_t n_vis = L - T + 2 + t;", ATTN_PINS),
    ("scale dropped", "        s *= J->sm_scale;", "        s *= 1.0;", ATTN_PINS),
    ("values read from K", "o[c] += w * kv_elem(J->v_cache, J->kv_dtype, J->v_scale",
     "o[c] += w * kv_elem(J->k_cache, J->kv_dtype, J->k_scale", ATTN_PINS),
    ("softmax denominator dropped", "double w = score[p] / denom;", "double w = score[p];", ATTN_PINS),
    ("fp8 scale dropped", "* (double)scale[blk];", "* 1.0;", ATTN_PINS),
    ("bf16 bias off by one", "return sign * ldexp(1.0 + (double)m / 128.0, e - 127);",
     "return sign * ldexp(1.0 + (double)m / 128.0, e - 126);", ATTN_PINS),
    ("e4m3 subnormal exponent", "return sign * ldexp((double)m / 8.0, -6);",
     "return sign * ldexp((double)m / 8.0, -7);", ATTN_PINS),
    ("residual sign flipped", "double r = p[j] - (double)qrow[j];", "double r = (double)qrow[j] - p[j];", SAMPLE_PINS),
    ("residual is p itself", "double r = p[j] - (double)qrow[j];\n            w[j] = r > 0.0 ? r : 0.0;",
     "double r = p[j] - (double)qrow[j];\n            w[j] = p[j];", SAMPLE_PINS),
    ("acceptance ratio inverted", "if (!((double)u[i] * c < a)) {", "if (!((double)u[i] * a < c)) {", SAMPLE_PINS),
    ("non-strict acceptance", "if (!((double)u[i] * c < a)) {", "if (!((double)u[i] * c <= a)) {", SAMPLE_PINS),
    ("inverse CDF >=", "if (C > target) {", "if (C >= target) {", SAMPLE_PINS),
    ("final row always 0", "if (row_dist(J, b, n, p) && near < 0)", "if (row_dist(J, b, 0, p) && near < 0)", SAMPLE_PINS),
    ("bonus from draft-free row K-1",
     "        for (int64_t j = 0; j < V; ++j) {\n            w[j] = p[j];\n            S += w[j];\n        }\n    }\n    J->resid_mass",
     "        oracle_softmax_row(J->target_logits + ((int64_t)b * (K + 1) + K - 1) * V, V, p);\n        for (int64_t j = 0; j < V; ++j) {\n            w[j] = p[j];\n            S += w[j];\n        }\n    }\n    J->resid_mass",
     SAMPLE_PINS),
    ("bf16 ties away from zero", "if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))", "if (drop >= 0x8000u)", KV_PINS),
    ("e4m3 ties to odd", "if (d < bestd || (d == bestd && (c & 1) == 0)) {", "if (d < bestd || (d == bestd && (c & 1) == 1)) {", KV_PINS),
    ("e4m3 overflow to NaN", "    if (a >= 448.0)\n        return (uint8_t)(sign | 0x7E);", "    if (a > 464.0)\n        return (uint8_t)(sign | 0x7F);", KV_PINS),
    ("e4m3 scale multiplied", "float qf = x / scale;", "float qf = x * scale;", KV_PINS),
    ("append slot shifted", "int slot = p % 16;", "int slot = (p + 1) % 16;", KV_PINS),
    ("append K and V swapped", "const float x = which ? v_new[src] : k_new[src];", "const float x = which ? k_new[src] : v_new[src];", KV_PINS),
    ("rollback drops one more", "int L = context_lens[b] - K + num_accepted[b];", "int L = context_lens[b] - K - 1 + num_accepted[b];", KV_PINS),
    ("pages in use rounded down", "pages_in_use[b] = (L + 15) / 16;", "pages_in_use[b] = L / 16;", KV_PINS),
    ("temperature multiplies", "p[j] = exp(((double)logits[j] - m) / tau);", "p[j] = exp(((double)logits[j] - m) * tau);", TEMP_PINS),
    ("greedy takes the last maximum", "        if ((double)logits[j] > m) {\n            m = (double)logits[j];\n            arg = j;",
     "        if ((double)logits[j] >= m) {\n            m = (double)logits[j];\n            arg = j;", TEMP_PINS),
    ("temperature halved", "const double tau = J->temperature ? (double)J->temperature[b] : 1.0;\n    const float *lrow",
     "const double tau = J->temperature ? (double)J->temperature[b] * 0.5 : 1.0;\n    const float *lrow", TEMP_PINS),
    ("top-p not renormalised", "        p[j] /= kept;", "        p[j] /= 1.0;", TOPP_PINS),
    ("top-p splits ties", "while (e < V && r[e].l == r[g].l)", "while (e < V && e == g)", TOPP_PINS),
    ("top-p ranks ascending", "return x->l > y->l ? -1 : 1;", "return x->l < y->l ? -1 : 1;", TOPP_PINS),
    ("top-p may drop the top group", "const int keep = first || above < top_p;", "const int keep = above < top_p;", TOPP_PINS),
    ("top-p counts the token itself", "const int keep = first || above < top_p;",
     "const int keep = first || above + mass < top_p;", TOPP_PINS),
    ("tree: residual coefficient not accumulated", "            C += Z;\n        }\n        if (next < 0)",
     "            C = Z;\n        }\n        if (next < 0)", TREE_PINS),
    ("tree: siblings tested against p", "a = (Z > 0.0 && rx > 0.0) ? rx / Z : 0.0;", "a = p[x];", TREE_PINS),
    ("tree: final draw ignores the rejections", "double r = C == 0.0 ? p[j] : p[j] - C * (double)qrow[j];",
     "double r = p[j];", TREE_PINS),
    ("tree: attention ignores the ancestor sets",
     "!((anc >> (p - (L - T))) & 1u)) {\n            score[p] = -INFINITY;",
     "0) {\n            score[p] = -INFINITY;", TREE_PINS),
    ("tree: ancestor sets of the chain", "m[c] = m[par[c]] | (1u << c);", "m[c] = (2u << c) - 1u;", TREE_PINS),
    ("typical: entropy sign", "h -= p[j] * log(p[j]);", "h += p[j] * log(p[j]);", TYPICAL_PINS),
    ("typical: threshold takes the larger", "const double th = fmin(J->eps,", "const double th = fmax(J->eps,",
     TYPICAL_PINS),
    ("typical: exp(+H)", "J->delta * exp(-oracle_entropy(p, V))", "J->delta * exp(oracle_entropy(p, V))", TYPICAL_PINS),
    ("typical: non-strict comparison", "if (!(p[x] > th)) {", "if (!(p[x] >= th)) {", TYPICAL_PINS),
    ("typical: draw from the first row",
     "oracle_target_row(J->target_logits + ((int64_t)b * (K + 1) + n) * V, V, tau, p);\n    double S = 0.0;",
     "oracle_target_row(J->target_logits + ((int64_t)b * (K + 1) + 0) * V, V, tau, p);\n    double S = 0.0;",
     TYPICAL_PINS),
    ("tree commit: destinations one early", "const int ps = base + path[(int64_t)b * N + i], pd = base + 1 + i;",
     "const int ps = base + path[(int64_t)b * N + i], pd = base + i;", COMMIT_PINS),
    ("tree commit: length without the root", "context_lens[b] = base + 1 + n;", "context_lens[b] = base + n;",
     COMMIT_PINS),
    ("tree commit: E4M3 codes copied across pages", "if (kv_dtype != OR_KV_FP8_E4M3 || pgs == pgd) {",
     "if (1) {", COMMIT_PINS),
    ("max not subtracted properly", "p[j] = exp((double)logits[j] - m);", "p[j] = exp((double)logits[j] - m) + 1e-3;", SAMPLE_PINS),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    with tempfile.TemporaryDirectory() as tmp:
        path_c = os.path.join(tmp, "mutant.c")
        path_so = os.path.join(tmp, "libmutant.so")
        with open(path_c, "w") as f:
            f.write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", path_c, "-o", path_so,
                        "-lm", "-lpthread"], check=True)
        caught = False
        with oracle.use_library(path_so):
            for pin in pins:
                try:
                    pin()
                except (AssertionError, ValueError):
                    caught = True
                    break
        assert caught, "no pin caught the planted mistake: " + name
