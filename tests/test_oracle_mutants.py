"""Plant plausible mistakes in a copy of the oracle and check the pins catch
each one (CPU only; the real oracle is never modified).

Each mutant is a one-line text edit of `oracle/attention.py`, loaded as a
separate module and swapped into the `oracle` package while the pin checks
run. A mutant survives only if every pin still passes; then the pins would
not have noticed that mistake, and this test fails.
"""
import os
import types

import pytest

import oracle
import test_oracle_append as A
import test_oracle_merge as M
import test_oracle_multi as MM
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "strided_head_groups": ("hs = [h for h in range(g * n_rep, (g + 1) * n_rep)",
                            "hs = [h for h in range(g, h_q, h_kv)"),
    "scale_dropped": ("s = sc * (Qg @ Kg.T)", "s = (Qg @ Kg.T)"),
    "scale_inverted": ("s = sc * (Qg @ Kg.T)", "s = (Qg @ Kg.T) / sc"),
    "no_max_subtraction": ("# [r, S]\n            s -= s.max(axis=1, keepdims=True)", "# [r, S]\n            pass"),
    "not_normalised": ("p = e / e.sum(axis=1, keepdims=True)", "p = e"),
    "offsets_shifted": ("off[1:] = np.cumsum(lens[:-1])", "off[1:] = np.cumsum(lens[1:])"),
    "k_and_v_swapped": ("Kg = widen(k[off[b]:off[b] + S, g, :], dtype)          # [S, d]",
                        "Kg = widen(v[off[b]:off[b] + S, g, :], dtype)          # [S, d]"),
    "q_k_transposed": ("s = sc * (Qg @ Kg.T)", "s = sc * (Kg[:Qg.shape[0], :Qg.shape[0]] @ Qg)"),
    "empty_seq_not_zero": ("                out[b, hs, :] = 0.0", "                out[b, hs, :] = 1.0"),
    "bf16_widen_shift": ("bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
                         "bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(15)"),
    "merge_wrong_sign": ("f1 = math.exp(m1 - mc) if m1 != NEG_INF else 0.0",
                         "f1 = math.exp(mc - m1) if m1 != NEG_INF else 0.0"),
    "merge_drops_factor": ("return mc, l1 * f1 + l2 * f2, o1 * f1 + o2 * f2",
                           "return mc, l1 * f1 + l2 * f2, o1 * f1 + o2"),
    "merge_keeps_first_max": ("mc = max(m1, m2)", "mc = m1 if m1 != NEG_INF else m2"),
    "triplet_not_centred": ("e = np.exp(s - m)", "e = np.exp(s)"),
    "triplet_normalised_o": ("return m, float(e.sum()), e @ v_rows",
                             "return m, float(e.sum()), (e / e.sum()) @ v_rows"),
    "finalize_no_division": ("    return o / l", "    return o"),
    "fanout_forwards_merge": ("east = [inbox_w[i] if i < n - 1 else None for i in range(n)]",
                              "east = [state[i] if i < n - 1 else None for i in range(n)]"),
    "multi_causal_off_by_one": ("s = sc * (Qi @ Kg[:p + 1].T)", "s = sc * (Qi @ Kg[:p].T)"),
    "multi_position_from_start": ("p = S - S_q + i", "p = min(S - 1, i + S // 2)"),
    "multi_values_not_causal": ("out[b, i, hs, :] = (e / e.sum(axis=1, keepdims=True)) @ Vg[:p + 1]",
                                "out[b, i, hs, :] = (e / e.sum(axis=1, keepdims=True)) @ Vg[S - p - 1:]"),
    "scores_scale_dropped": ("return float(np.float32(scale)) * (k_rows @ q_row)", "return k_rows @ q_row"),
    "scores_sign_flipped": ("return float(np.float32(scale)) * (k_rows @ q_row)",
                            "return -float(np.float32(scale)) * (k_rows @ q_row)"),
    "append_one_row_late": ("pos = int(lens[b]) + i", "pos = int(lens[b]) + i + 1"),
    "append_lengths_not_clamped": ("np.minimum(lens + n_new, capacity)", "(lens + n_new)"),
    "append_k_into_v": ("vc[off + pos] = v_new[b, i]", "vc[off + pos] = k_new[b, i]"),
    "fanout_east_first": ("            if inbox_w[i] is not None:\n                state[i] = merge(state[i], inbox_w[i])\n                order[i].append(inbox_w_org[i])\n            if inbox_e[i] is not None:\n                state[i] = merge(state[i], inbox_e[i])\n                order[i].append(inbox_e_org[i])",
                          "            if inbox_e[i] is not None:\n                state[i] = merge(state[i], inbox_e[i])\n                order[i].append(inbox_e_org[i])\n            if inbox_w[i] is not None:\n                state[i] = merge(state[i], inbox_w[i])\n                order[i].append(inbox_w_org[i])"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique or missing"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


def pin_checks():
    """The pin tests as zero-argument callables (one instance per pin)."""
    ex = {e["name"]: e for e in
          __import__("json").load(open(os.path.join(P.GOLDEN, "closed_form_examples.json")))["examples"]}
    c = [lambda s=s: P.test_oracle_matches_brute_force(*s) for s in P.SHAPES]
    c += [lambda e=e: P.test_closed_form_examples(e) for e in ex.values()]
    c += [P.test_oracle_on_bf16_bits_matches_brute_force, P.test_widen_bf16_is_exact,
          P.test_single_token_gives_its_value_row, P.test_equal_scores_give_mean_of_values,
          P.test_identical_value_rows_give_that_row, P.test_one_hot_dominant_score_selects_its_row,
          P.test_large_scores_stay_finite_and_exact, P.test_head_mapping_is_contiguous_groups,
          P.test_token_offsets_follow_packed_layout, P.test_ragged_batch_equals_independent_sequences,
          P.test_shift_of_all_scores_changes_nothing, P.test_output_inside_value_hull,
          P.test_scores_on_hand_values, P.test_scores_triplet_finalize_is_brute_force]
    c += [lambda: M.test_whole_triplet_equals_unsplit(17),
          lambda: M.test_random_chunkings_with_empty_chunks(257, 8, 1),
          M.test_size_one_chunks_every_order, M.test_tree_merge_equals_sequential,
          M.test_merge_formula_on_hand_values, M.test_empty_triplets,
          M.test_merge_survives_far_apart_maxima,
          lambda: M.test_fanout_every_rank_gets_the_unsplit_answer(5),
          lambda: M.test_fanout_arrival_step_is_rank_distance(4),
          M.test_triplet_matches_definition]
    c += [MM.test_single_query_token_is_attend, lambda: MM.test_each_token_is_brute_force_on_its_prefix(3),
          MM.test_future_positions_do_not_matter, MM.test_last_token_sees_everything,
          MM.test_more_query_tokens_than_cached_positions]
    c += [A.test_rows_land_where_expected, A.test_explicit_offsets,
          A.test_append_then_attend_equals_attend_on_full_cache]
    return c


NAMES = ["NEG_INF", "attend", "attend_multi", "fanout", "finalize", "kv_append", "merge", "scores",
         "token_offsets", "triplet", "widen"]


def test_every_exported_function_is_swapped():
    """Every name the oracle package exports is replaced by the mutant's, so a
    mistake planted in any exported function reaches the pins."""
    assert sorted(NAMES) == sorted(oracle.__all__)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    mod = load_mutant(name)
    for n in NAMES:
        monkeypatch.setattr(oracle, n, getattr(mod, n))
    caught = 0
    for check in pin_checks():
        try:
            check()
        except Exception:  # any failure of a pin counts as detection
            caught += 1
    assert caught > 0, f"no pin fails for planted mistake {name!r}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    mod = types.ModuleType("oracle_copy")
    exec(compile(open(SRC).read(), SRC, "exec"), mod.__dict__)
    for n in NAMES:
        monkeypatch.setattr(oracle, n, getattr(mod, n))
    for check in pin_checks():
        check()
