"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's source (on the
CPU; the real oracle is untouched), rebinds the pin tests to the mutant and
requires at least one pin to fail.  This shows the pins are not satisfied by
a wrong oracle: a flipped residual sign, a reused uniform, a shifted slot
index, a transposed acceptance ratio, a dropped temperature, an off-by-one
top-k, a non-strict inverse CDF, a wrong greedy replacement, or in the relaxed
rule a dropped factor in gamma, a rank that counts ties or an off-by-one
rank guard, and in the tree walk a residual taken from the target instead of
the last residual, a residual left unnormalised, siblings tested against the
target instead of the residual, a final draw from the target or a greedy walk
that ignores the argmax.  The batch wrappers are covered too (a shifted row
index, a greedy row whose draft is read), as are the margins (a margin taken
over positions the scan never reached, or without the final draw), the forced
outcomes tests use to follow the other side of a near decision, and the set
of draws near the sampled point.
"""

from __future__ import annotations

import sys
import types

import pytest

import oracle.verifier as ov
import tests.test_oracle_pins as pins

SRC = open(ov.__file__).read()

MUTANTS = {
    "residual_sign": ("w = np.maximum(0.0, P[n] - Q[n])", "w = np.maximum(0.0, Q[n] - P[n])"),
    "reuse_u_n": ("    t = u[K] * S\n    x, gap", "    t = u[n] * S\n    x, gap"),
    "shifted_target_slot": ("p_d[i] = P[i][tok]", "p_d[i] = P[min(i + 1, K)][tok]"),
    "transposed_ratio": ("accept[i] = u[i] * q_d[i] < p_d[i]", "accept[i] = u[i] * p_d[i] < q_d[i]"),
    "draft_without_temperature": ("Q.append(tempered_softmax(np.where(keep, dl[i], -np.inf), T))",
                                  "Q.append(tempered_softmax(np.where(keep, dl[i], -np.inf), 1.0))"),
    "bonus_wrong_slot": ("        w = P[K]\n", "        w = P[max(K - 1, 0)]\n"),
    "topk_off_by_one": ("keep[order[:k]] = True", "keep[order[:k + 1]] = True"),
    "topk_ties_highest_id": ("order = np.argsort(-logits, kind=\"stable\")",
                             "order = (V - 1 - np.argsort(-logits[::-1], kind=\"stable\"))"),
    "cdf_not_strict": ("above = np.flatnonzero(C > t)", "above = np.flatnonzero(C >= t)"),
    "temperature_multiplies": ("z = np.asarray(logits, dtype=np.float64) / float(T)",
                               "z = np.asarray(logits, dtype=np.float64) * float(T)"),
    "greedy_keeps_draft": ("        tokens[n] = a[n]\n", "        tokens[n] = d[n] if n < K else a[n]\n"),
    "greedy_tie_highest_id": ("a = [int(np.argmax(tl[i])) for i in range(K + 1)]",
                              "a = [int(V - 1 - np.argmax(tl[i][::-1])) for i in range(K + 1)]"),
    "residual_unclipped": ("w = np.maximum(0.0, P[n] - Q[n])", "w = np.abs(P[n] - Q[n])"),
    "gamma_without_factor_two": ("np.sqrt(2.0 * alpha * p * (1.0 - p))", "np.sqrt(alpha * p * (1.0 - p))"),
    "rank_counts_ties": ("1 + int(np.count_nonzero(logits > logits[tok]))",
                         "1 + int(np.count_nonzero(logits >= logits[tok]))"),
    "kl_reversed": ("return float(np.sum(P[m] * (np.log(P[m]) - np.log(Q[m]))))",
                    "return float(np.sum(Q[m] * (np.log(Q[m]) - np.log(P[m]))))"),
    "kl_without_temperature": ("    P = tempered_softmax(target_logits, T)\n    Q = tempered_softmax(draft_logits, T)",
                               "    P = tempered_softmax(target_logits, 1.0)\n    Q = tempered_softmax(draft_logits, 1.0)"),
    "tree_residual_from_target": ("            res = np.maximum(0.0, r - Q)",
                                  "            res = np.maximum(0.0, P - Q)"),
    "tree_residual_not_normalised": ("            r = res / m\n", "            r = res\n"),
    "tree_siblings_against_target": ("pd, qd, rd = (P[d], Q[d], r[d])", "pd, qd, rd = (P[d], Q[d], P[d])"),
    "tree_final_from_target": ("        else:\n            w = r\n        break", "        else:\n            w = P\n        break"),
    "tree_descends_first_child": ("            nxt = next((c for c in ch[v] if int(tok[c]) == a), None)",
                                  "            nxt = ch[v][0] if ch[v] else None"),
    "verify_shifted_row": ("        tl = decode_logits(target_raw[b], dtype)\n        T = float(temperature[b])",
                           "        tl = decode_logits(target_raw[(b + 1) % B], dtype)\n        T = float(temperature[b])"),
    "verify_greedy_reads_draft": ("        if K > 0 and T > 0:\n            dl = decode_logits(draft_raw[b], dtype)",
                                  "        if K > 0:\n            dl = decode_logits(draft_raw[b], dtype)"),
    "verify_tree_shifted_row": ("        tl = decode_logits(target_raw[b], dtype)\n        dl = decode_logits(draft_raw[b], dtype) if T",
                                "        tl = decode_logits(target_raw[(b + 1) % B], dtype)\n        dl = decode_logits(draft_raw[b], dtype) if T"),
    "verify_tree_greedy_reads_draft": ("dl = decode_logits(draft_raw[b], dtype) if T > 0 else None",
                                       "dl = decode_logits(draft_raw[b], dtype)"),
    "margin_over_unreached": ("reached = self.margins[: min(self.n + 1, K)]", "reached = self.margins"),
    "margin_without_draw": ("        return min(m, self.gap)", "        return m"),
    "tree_margin_without_draw": ("return min(min(self.margins, default=float(\"inf\")), self.gap)",
                                 "return min(self.margins, default=float(\"inf\"))"),
    "force_ignored": ("        taken[int(i)] = bool(outcome)", "        pass"),
    "near_ids_only_the_draw": ("(starts <= t + draw_eps) & (C >= t - draw_eps)", "(starts <= t) & (C > t)"),
    "guard_ignores_rank": ("if relaxed.max_rank > 0 and ranks[i] > relaxed.max_rank:",
                           "if relaxed.max_rank > 0 and ranks[i] > relaxed.max_rank + 1:"),
}


def _mutant_module(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = ov.__file__
    sys.modules[mod.__name__] = mod        # dataclasses resolve annotations through it
    try:
        exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


def _run_pins():
    """Run a fixed list of pins; return how many fail."""
    cases = [
        lambda: pins.test_lossless_enumeration(5, 3, 1.0, 0, 1),
        lambda: pins.test_lossless_enumeration(6, 3, 0.8, 3, 4),
        lambda: pins.test_lossless_enumeration(6, 0, 0.9, 0, 6),
        lambda: pins.test_greedy_equals_greedy_decode_prefix(5, 3, 11),
        pins.test_greedy_argmax_tie_lowest_id_and_ignores_uniforms,
        pins.test_early_rejection_golden,
        pins.test_softmax_closed_forms,
        lambda: pins.test_topk_matches_brute_force_rank(5),
        pins.test_topk_ties_lowest_id_and_degenerate_k,
        pins.test_zero_weight_token_never_emitted_at_u_zero,
        pins.test_k0_is_textbook_inverse_cdf,
        pins.test_residual_never_picks_token_where_p_le_q,
        lambda: pins.test_relaxed_acceptance_probability(0.5, 0.2, 0.8, 0.75),
        lambda: pins.test_relaxed_acceptance_probability(2.0, 0.5, 0.6, 1.0),
        pins.test_target_rank_brute_force,
        pins.test_support_guard,
        pins.test_kl_two_token_closed_form,
        pins.test_kl_properties,
        lambda: pins.test_tree_lossless_enumeration("fan2", 4, 1.0, 0, 41),
        lambda: pins.test_tree_lossless_enumeration("binary2", 4, 1.2, 0, 43),
        pins.test_tree_greedy_is_greedy_decode,
        lambda: pins.test_verify_batch_equals_rows_and_skips_greedy_drafts(0),
        pins.test_verify_tree_batch_equals_rows_and_skips_greedy_drafts,
        pins.test_min_margin_takes_reached_decisions_and_the_draw,
        pins.test_tree_min_margin_takes_tested_nodes_and_the_draw,
        pins.test_forced_outcome_follows_the_other_path,
        pins.test_near_ids_are_the_neighbours_of_t,
    ]
    failed = 0
    for c in cases:
        try:
            c()
        except Exception:
            failed += 1
    return failed


def test_unmutated_oracle_passes_the_pin_set():
    assert _run_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    mod = _mutant_module(name)
    for attr in ("verify_row", "tempered_softmax", "topk_keep_mask", "decode_logits"):
        monkeypatch.setattr(pins, attr, getattr(mod, attr))
    # The relaxed-rule pins reach these through the oracle package.
    for attr in ("Relaxed", "target_rank", "relaxed_gamma", "kl_divergence", "verify_tree_row",
                 "tree_children", "verify", "verify_tree", "verify_row"):
        monkeypatch.setattr(pins.oracle, attr, getattr(mod, attr))
    assert _run_pins() > 0, f"no pin caught the planted mistake {name!r}"
