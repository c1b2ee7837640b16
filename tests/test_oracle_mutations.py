"""Planted mistakes in the oracle (CPU only): each must make at least one pin fail.

Every case swaps one step of the oracle for a plausible wrong version -- a dropped
term, a flipped ratio, a wrong index -- and runs the pin that is meant to catch it."""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.chain as ochain
import oracle.proj as oproj
import oracle.verify as over
from tests import test_oracle_attention as t_att
from tests import test_oracle_chain as t_chain
from tests import test_oracle_proj as t_proj
from tests import test_oracle_verify as t_ver


def fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_flipped_acceptance_ratio_is_caught(monkeypatch):
    monkeypatch.setattr(over, "acceptance_probability", lambda P, Q: 1.0 if Q >= P else Q / P)
    fails(t_ver.test_emitted_token_follows_anchor_distribution, "random")


def test_wrong_residual_is_caught(monkeypatch):
    monkeypatch.setattr(over, "residual_weights", lambda p, q: np.maximum(0.0, q - p))
    fails(t_ver.test_residual_matches_hand_computation)


def test_residual_without_q_subtraction_is_caught(monkeypatch):
    monkeypatch.setattr(over, "residual_weights", lambda p, q: np.maximum(0.0, p))
    fails(t_ver.test_emitted_token_follows_anchor_distribution, "random")


def test_unrescaled_residual_uniform_is_caught(monkeypatch):
    monkeypatch.setattr(over, "residual_uniform", lambda u, a: u)
    fails(t_ver.test_emitted_token_follows_anchor_distribution, "random")


def test_highest_id_on_ties_is_caught(monkeypatch):
    monkeypatch.setattr(over, "argmax_lowest", lambda raw: int(np.flatnonzero(raw == raw.max())[-1]))
    fails(t_ver.test_argmax_lowest_id_on_ties)


def test_inverse_cdf_off_by_one_is_caught(monkeypatch):
    orig = over.inverse_cdf

    def shifted(w, u):
        k, lo, hi = orig(w, u)
        return min(k + 1, len(w) - 1), lo, hi
    monkeypatch.setattr(over, "inverse_cdf", shifted)
    fails(t_ver.test_samples_and_bonus_match_brute_force)


def test_causal_diagonal_dropped_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "causal_extent", lambda L, r: L + r)
    fails(t_att.test_attention_matches_brute_force, 5, 2, 4, 8, 2, 8, [5, 17], "f32")


def test_bidirectional_block_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "causal_extent", lambda L, r: L + 7)
    fails(t_att.test_row_sees_itself_but_not_later_rows)


def test_wrong_page_slot_is_caught(monkeypatch):
    def gather(pages, row, n):
        j = np.arange(n)
        return oracle.stored.to_f64(pages[row[j // 16], :, (j + 1) % 16, :])
    monkeypatch.setattr(oatt, "gather_keys", gather)
    fails(t_att.test_attention_matches_brute_force, 2, 2, 4, 4, 2, 16, [0, 40], "f32")


def test_missing_lowrank_rounding_is_caught(monkeypatch):
    monkeypatch.setattr(oproj, "round_bf16", lambda x: x)
    fails(t_proj.test_gated_proj_matches_brute_force)


def test_wrong_tpf_exponent_is_caught(monkeypatch):
    monkeypatch.setattr(ochain, "tpf_closed_form",
                        lambda N, p: (2 + sum(p ** k for k in range(1, N - 1))) / (2 - p ** N))
    fails(t_chain.test_printed_tpf_and_efficiency, {
        "tpf_n4_p09": {"N": 4, "p": 0.9, "value": 2.9, "decimals": 1},
        "efficiency_n4_p09": {"N": 4, "p": 0.9, "queries": 7, "value": 1.22, "decimals": 2},
        "queries_per_forward_n4": {"value": 7}})


def test_lm_head_without_rounding_is_caught(monkeypatch):
    import oracle.lm_head as olm
    from tests import test_oracle_lm_head as t_lm
    monkeypatch.setattr(olm, "round_bf16", lambda x: x)
    fails(t_lm.test_grid_inputs_give_the_exact_product_rounded_to_bf16)


def test_lm_head_wrong_weight_column_is_caught(monkeypatch):
    import oracle.lm_head as olm
    from tests import test_oracle_lm_head as t_lm
    monkeypatch.setattr(olm, "lm_head_logits",
                        lambda h, w: olm.round_bf16(olm.to_f64(h) @ np.roll(olm.to_f64(w), 1, axis=1).T))
    fails(t_lm.test_one_hot_rows_pick_one_weight_each)


def test_layer_sigmoid_for_silu_is_caught(monkeypatch):
    import oracle.layer as olay
    from tests import test_oracle_layer as t_lay
    monkeypatch.setattr(olay, "silu", lambda z: 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64))))
    fails(t_lay.test_layer_matches_brute_force, 11, True)


def test_layer_dropped_residual_is_caught(monkeypatch):
    import oracle.layer as olay
    from tests import test_oracle_layer as t_lay
    monkeypatch.setattr(olay, "residual", lambda x, y: olay.round_bf16(y))   # h = o(att), no x
    fails(t_lay.test_layer_matches_brute_force, 12, True)


def test_layer_swapped_gate_and_up_is_caught(monkeypatch):
    import oracle.layer as olay
    from tests import test_oracle_layer as t_lay
    orig = olay.linear
    swap = {"gate": "up", "up": "gate"}
    monkeypatch.setattr(olay, "linear", lambda y, w, name, g: orig(y, w, swap.get(name, name), g))
    fails(t_lay.test_layer_matches_brute_force, 11, True)
