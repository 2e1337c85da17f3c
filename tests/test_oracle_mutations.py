"""The oracle's pins are sensitive: each plausible mistake planted in the oracle (on the CPU, through
monkeypatching) makes at least one pin check fail."""
import math

import numpy as np
import pytest

import oracle as O
from oracle import pisa_oracle as PO

import test_oracle_pins as P


def _pins_pass() -> bool:
    checks = [
        lambda: P.test_walk_equals_flat_exact_when_k_covers_level1(16),
        lambda: P.test_walk_equals_dense_two_level_bruteforce(5, 2),
        lambda: P.test_walk_monotone_keys_closed_form(+1, 1000),
        lambda: P.test_walk_monotone_keys_closed_form(-1, 1000),
        lambda: P.test_pyramid_recursive_equals_direct_span_mean(1000, 32),
        lambda: P.test_attention_all_blocks_equals_dense_sdpa(),
        lambda: P.test_selection_invariants(),
        lambda: P.test_exact_ties_break_to_lowest_index(4),
        lambda: P.test_sel_lse_equals_library_lse_over_selected_tokens(3, "ar1"),
        lambda: P.test_walk_equals_dense_all_levels_bruteforce(4, 2),
        lambda: P.test_bsa_matches_dense_mean_key_scores(),
        lambda: P.test_row_lse_and_mass_closed_forms(),
        lambda: P.test_mass_equals_leaf_lse_weights(),
        lambda: P.test_pooled_summaries_closed_forms(1000),
        lambda: P.test_mean_scoring_with_k_covering_level1_is_flat_bsa(),
        lambda: P.test_mean_var_scoring_equals_dense_formula(),
        lambda: P.test_halving_budget_and_truncation_equal_dense_bruteforce(3, 1),
        lambda: P.test_backward_equals_autograd_of_dense_masked_attention(),
        lambda: P.test_backward_finite_differences(),
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_unmutated_oracle_passes():
    assert _pins_pass()


def _mut_topk_ascending(cands, scores):
    return sorted(range(len(cands)), key=lambda p: (scores[p], cands[p]))


def _mut_tiebreak_high_index(cands, scores):
    return sorted(range(len(cands)), key=lambda p: (-scores[p], -cands[p]))


def _mut_leaf_no_causal_mask(qg, k, j, i, C, scale, n_tokens):
    t0, t1 = j * C, min(n_tokens, (j + 1) * C)
    return O.logsumexp(scale * (qg @ k[t0:t1].T), axis=-1)


def _mut_node_uses_max(qg, pyr, l, j, i, scale):
    kids = [c for c in PO.children(l, j, pyr) if PO.eligible(l - 1, c, i, pyr.C, pyr.g)]
    return np.max(scale * (qg @ pyr.means[l - 1][kids].T), axis=-1)


def _mut_node_ignores_eligibility(qg, pyr, l, j, i, scale):
    kids = PO.children(l, j, pyr)
    return O.logsumexp(scale * (qg @ pyr.means[l - 1][kids].T), axis=-1)


def _mut_children_shifted(l, j, pyr):
    n_prev = pyr.means[l - 1].shape[0]
    return [c for c in range(j * pyr.g + 1, (j + 1) * pyr.g + 1) if c < n_prev]


_orig_build = PO.build_pyramid


def _mut_pyramid_sums(k, C, g=2, n_tokens=None):
    p = _orig_build(k, C, g, n_tokens)
    p.means = [m * c[:, None] for m, c in zip(p.means, p.counts)]
    return p


def _mut_pyramid_unweighted(k, C, g=2, n_tokens=None):
    p = _orig_build(k, C, g, n_tokens)
    for l in range(1, len(p.means)):
        prev = p.means[l - 1]
        for j in range(p.means[l].shape[0]):
            kids = list(range(j * g, min((j + 1) * g, prev.shape[0])))
            p.means[l][j] = prev[kids].mean(axis=0)
    return p


_orig_scale_attend = PO.attend_unit


def _mut_attend_no_scale(qg, k, v, sel, i, C, scale, n_tokens):
    return _orig_scale_attend(qg, k, v, sel, i, C, 1.0, n_tokens)


def _mut_margin_max_over_levels(level_margins):
    return max(level_margins.values(), default=math.inf)


def _mut_margin_leaf_level_only(level_margins):
    return level_margins.get(0, math.inf)


def _mut_margin_off_by_one_rank(scores, order, K):
    return scores[order[K]] - scores[order[K + 1]] if len(order) > K + 1 else math.inf


def _mut_sel_lse_reversed(active, leaf_head_lse, G, K):
    out = np.full((G, K), -np.inf)
    for s_, j in enumerate(reversed(active)):
        out[:, s_] = leaf_head_lse[j]
    return out


_orig_mass = PO.attention_mass_unit


def _mut_mass_past_i(qg, k, sel, i, C, scale):
    # the selected leaves' tokens after i are counted too (the mass then exceeds the causal share)
    return _orig_mass(qg, k, np.array([j for j in sel]), min(k.shape[0] - 1, i + C), C, scale)


def _mut_row_lse_without_diagonal(qg, k, i, scale):
    return O.logsumexp(scale * (np.asarray(qg) @ k[:i].T), axis=-1) if i > 0 else \
        O.logsumexp(scale * (np.asarray(qg) @ k[:1].T), axis=-1)


_orig_vscore = PO.variant_node_score


def _mut_var_term_without_half(qg, pyr, l, j, i, scale, score, k, variances=None):
    x = _orig_vscore(qg, pyr, l, j, i, scale, score, k, variances)
    if score == "mean_var":
        x += float((0.5 * scale * scale * ((qg * qg) @ variances[l][j])).sum())
    return x


def _mut_budget_one_level_off(l, n_l, K, budget):
    # the doubling starts one level late: K at levels 0 and 1, then K 2^(l-1)
    return K if budget == "fixed" or l == 0 else min(n_l, K * 2 ** (l - 1))


_orig_pooled = PO.build_pyramid_pooled


def _mut_max_pool_is_mean(k, C, g=2, pool="mean", n_tokens=None):
    return _orig_pooled(k, C, g, "mean" if pool == "max" else pool, n_tokens)


_orig_variant = PO.select_unit_variant


def _mut_truncation_one_level_high(qg, k, pyr, i, K, scale, score="lse", budget="fixed", max_level=None,
                                   variances=None):
    return _orig_variant(qg, k, pyr, i, K, scale, score, budget, None if max_level is None else max_level + 1,
                         variances)


def _mut_mean_score_uses_lse(qg, pyr, l, j, i, scale, score, k, variances=None):
    return _orig_vscore(qg, pyr, l, j, i, scale, "lse" if score == "mean" else score, k, variances)


_orig_bwd = PO.attention_backward_head


def _mut_bwd_dk_unscaled(qg, k, v, sel, C, scale, do):
    dq, dk, dv = _orig_bwd(qg, k, v, sel, C, scale, do)
    return dq, dk / scale, dv


def _mut_bwd_dv_head_mean(qg, k, v, sel, C, scale, do):
    dq, dk, dv = _orig_bwd(qg, k, v, sel, C, scale, do)
    return dq, dk, dv / qg.shape[0]


MUTANTS = {
    "topk_ascending": ("_topk_order", _mut_topk_ascending),
    "tiebreak_high_index": ("_topk_order", _mut_tiebreak_high_index),
    "leaf_no_causal_mask": ("leaf_lse_per_head", _mut_leaf_no_causal_mask),
    "node_score_max": ("node_lse_per_head", _mut_node_uses_max),
    "node_ignores_eligibility": ("node_lse_per_head", _mut_node_ignores_eligibility),
    "children_off_by_one": ("children", _mut_children_shifted),
    "pyramid_sums_not_means": ("build_pyramid", _mut_pyramid_sums),
    "pyramid_unweighted_ragged": ("build_pyramid", _mut_pyramid_unweighted),
    "attention_without_scale": ("attend_unit", _mut_attend_no_scale),
    "margin_max_over_levels": ("_unit_margin", _mut_margin_max_over_levels),
    "margin_leaf_level_only": ("_unit_margin", _mut_margin_leaf_level_only),
    "margin_off_by_one_rank": ("_level_margin", _mut_margin_off_by_one_rank),
    "sel_lse_misaligned_with_sel": ("_selected_lse", _mut_sel_lse_reversed),
    "mass_counts_tokens_past_i": ("attention_mass_unit", _mut_mass_past_i),
    "row_lse_without_diagonal": ("row_lse_unit", _mut_row_lse_without_diagonal),
    "variance_term_doubled": ("variant_node_score", _mut_var_term_without_half),
    "halving_budget_one_level_off": ("level_budget", _mut_budget_one_level_off),
    "max_pooling_as_mean": ("build_pyramid_pooled", _mut_max_pool_is_mean),
    "truncation_one_level_high": ("select_unit_variant", _mut_truncation_one_level_high),
    "mean_scoring_as_lse": ("variant_node_score", _mut_mean_score_uses_lse),
    "backward_dk_unscaled": ("attention_backward_head", _mut_bwd_dk_unscaled),
    "backward_dv_head_mean": ("attention_backward_head", _mut_bwd_dv_head_mean),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(PO, attr, fn)
    monkeypatch.setattr(O, attr, fn, raising=False)
    assert not _pins_pass(), f"mutant {name} survived every pin"
