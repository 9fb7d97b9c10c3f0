"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each.

Each mutant is the oracle's own source with one textual edit, loaded as a
separate module; the real oracle is never modified.  A mutant "survives" if
every listed pin still passes — that would mean the pins do not cover it.
"""

import importlib.util
import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "flex_oracle.py")

# (name, original text, mutated text, pins expected to catch it)
MUTANTS = [
    ("drop_scale", "S = (Q @ K.T) * scale", "S = (Q @ K.T)",
     [lambda: pins.test_oracle_matches_sdpa_boolean_masks(16, "causal")]),
    ("mod_before_scale", "Sp[M] = score_mod(S[M], b, hq, qb[M], kb[M])",
     "Sp[M] = scale * score_mod(S[M] / scale, b, hq, qb[M], kb[M])",
     [lambda: pins.test_oracle_matches_sdpa_additive_mods("alibi")]),
    ("gqa_modulo", "hkv = hq // group", "hkv = hq % Hkv",
     [lambda: pins.test_oracle_matches_sdpa_boolean_masks(16, "none")]),
    ("alibi_sign", "s + sl[h] * (kv - q)", "s + sl[h] * (q - kv)",
     [lambda: pins.test_alibi_geometric_closed_form(4)]),
    ("alibi_slope_offset", "-8.0 * (h + 1) / H", "-8.0 * h / H",
     [pins.test_alibi_default_slopes_are_geometric]),
    ("softcap_inner_scale", "cap * np.tanh(s / cap)", "cap * np.tanh(s)",
     [pins.test_softcap_closed_form_and_limits]),
    ("rel_pos_sign", "s + (q - kv)", "s + (kv - q)",
     [pins.test_rel_pos_geometric_closed_form]),
    ("mask_as_zero", "Sp = np.full(S.shape, NEG_INF)", "Sp = np.full(S.shape, 0.0)",
     [lambda: pins.test_causal_row0_is_v0("none")]),
    ("lse_log2", "lse[live] = m[live] + np.log(l)", "lse[live] = m[live] + np.log2(l)",
     [pins.test_equal_scores_lse_is_log_count]),
    ("window_exclusive", "(q - kv) <= window", "(q - kv) < window",
     [pins.test_sliding_window_zero_is_identity_on_v, pins.test_mask_limits]),
    ("window_two_sided", "(q - kv) <= window", "abs(q - kv) <= window",
     [lambda: pins.test_oracle_matches_brute_force("sliding_window2", "none"),
      lambda: pins.test_oracle_matches_sdpa_boolean_masks(16, "window")]),
    ("attended_count_ragged_chunk", "qi = np.arange(r0, min(Sq, r0 + chunk), dtype=np.int64)[:, None]",
     "qi = np.arange(r0, r0 + chunk, dtype=np.int64)[:, None]",
     [lambda: pins.test_attended_count_closed_forms(64)]),
    ("decode_mod_ignores_position", "return score_mod(s, b, h, qi + pos[b], kv)", "return score_mod(s, b, h, qi, kv)",
     [lambda: pins.test_decode_at_query_positions_matches_sdpa("alibi"),
      pins.test_decode_at_position_p_is_row_p_of_the_causal_forward]),
    ("ragged_area", "area = (q1 - q0) * (k1 - k0)", "area = block * block",
     [lambda: pins.test_block_classes_brute_force(37, 50, "none")]),
    ("descending_lists", "cols = np.nonzero(flat_sel[r])[0]", "cols = np.nonzero(flat_sel[r])[0][::-1]",
     [pins.test_golden_causal_256]),
    ("prefix_exclusive_of_causal", "return or_masks(prefix(prefix_len), causal())",
     "return prefix(prefix_len)", [pins.test_mask_limits]),
    ("doc_ignores_batch", "doc[b, q] == doc[b, kv]", "doc[0, q] == doc[0, kv]",
     [lambda: pins.test_oracle_matches_sdpa_boolean_masks(16, "document")]),
    ("bwd_drop_softmax_jacobian_term", "dSp = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dSp = P * dP",
     [lambda: pins.test_backward_matches_torch_autograd_sdpa("causal")]),
    ("bwd_ignore_mod_derivative", "dS = dSp * grad_mod", "dS = dSp * (grad_mod != 0)",
     [pins.test_backward_softcap_matches_torch_autograd]),
    ("bwd_dq_unscaled", "dQ[b, hq] = scale * (dS @ K)", "dQ[b, hq] = dS @ K",
     [lambda: pins.test_backward_matches_torch_autograd_sdpa("none")]),
    ("bwd_dk_untransposed", "dK[b, hkv] += scale * (dS.T @ Q)", "dK[b, hkv] += scale * (dS @ Q)",
     [lambda: pins.test_backward_matches_torch_autograd_sdpa("alibi_causal")]),
    ("bwd_dv_overwrites_group", "dV[b, hkv] += P.T @ dO", "dV[b, hkv] = P.T @ dO",
     [pins.test_backward_gqa_equals_mha_summed_over_the_group]),
    ("bwd_unnormalised_p", "P[live] = E / E.sum(axis=1, keepdims=True)", "P[live] = E",
     [lambda: pins.test_backward_matches_finite_differences("causal", "none")]),
    ("transposed_lists_of_full_tiles", "q_num, q_idx = _compact(np.swapaxes(kv_sel, -1, -2))",
     "q_num, q_idx = _compact(np.swapaxes(full, -1, -2))", [pins.test_transposed_block_lists]),
]


def _mutant(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = types.ModuleType(spec.name)
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, old, new, checks):
    for check in checks:
        check()  # the real oracle passes the pin
    monkeypatch.setattr(pins, "fo", _mutant(name, old, new))
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught == len(checks), f"mutant {name} survived its pins"
