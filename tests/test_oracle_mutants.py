"""Each plausible mistake, planted in a copy of the oracle's source on the CPU,
must make at least one pin fail. The real oracle is never modified."""
import importlib.util
import os
import sys
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_oracle.py")

MUTANTS = {
    "softmax_scores": ("score = 1.0 / (1.0 + np.exp(-logits))",
                       "score = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)"),
    "gate_from_biased_choice": ("s_sel = np.take_along_axis(score, idx.astype(np.int64), axis=1)\n    gate",
                                "s_sel = np.take_along_axis(choice, idx.astype(np.int64), axis=1)\n    gate"),
    "no_renormalisation": ("gate = (routed_scaling * s_sel / s_sel.sum(axis=1, keepdims=True)).astype(np.float32)\n    return RouteResult",
                           "gate = (routed_scaling * s_sel).astype(np.float32)\n    return RouteResult"),
    "no_scaling": ("gate = (routed_scaling * s_sel / s_sel.sum(axis=1, keepdims=True)).astype(np.float32)\n    return RouteResult",
                   "gate = (s_sel / s_sel.sum(axis=1, keepdims=True)).astype(np.float32)\n    return RouteResult"),
    "bias_ignored": ("choice = score + b[None, :]", "choice = score + 0.0 * b[None, :]"),
    "bias_subtracted": ("choice = score + b[None, :]", "choice = score - b[None, :]"),
    "tie_to_higher_index": ("np.lexsort((admitted, -c[admitted]))", "np.lexsort((-admitted, -c[admitted]))"),
    "top_k_plus_one": ("chosen = order[:K]", "chosen = order[1:K + 1] if K < len(order) else order[:K]"),
    "gap_wrong_neighbour": ("c[order[K]] if K < len(order)", "c[order[min(K + 1, len(order) - 1)]] if K < len(order)"),
    "group_top1": ("[::-1][:2].sum()", "[::-1][:1].sum()"),
    "group_sum_all": ("np.sort(c[g * G:(g + 1) * G])[::-1][:2].sum()", "c[g * G:(g + 1) * G].sum()"),
    "group_score_unbiased": ("np.sort(c[g * G:(g + 1) * G])", "np.sort(score[t][g * G:(g + 1) * G])"),
    "group_tie_to_higher": ("np.lexsort((groups, -gs))", "np.lexsort((-groups, -gs))"),
    "group_one_too_many": ("gorder[:topk_group]]", "gorder[:topk_group + 1]]"),
    "group_gap_ignored": ("gap[t] = min(egap, ggap)", "gap[t] = egap"),
    "relu_not_squared": ("return r * r", "return r"),
    "no_activation": ("r = np.maximum(a, 0.0)\n    return r * r", "return a"),
    "shared_dropped": ("+ hs @ dec(w_sh_down_bits).T)", ")"),
    "shared_not_squared": ("hs = rnd(_relu2(x @ dec(w_sh_up_bits).T))",
                           "hs = rnd(np.maximum(x @ dec(w_sh_up_bits).T, 0))"),
    "combine_first_slot_only": ("y[p.slot_row[:, j]]", "y[p.slot_row[:, 0]]"),
    "gate_squared": ("gate64[:, j:j + 1] * y", "gate64[:, j:j + 1] ** 2 * y"),
    "gate_dropped_in_combine": ("gate64[:, j:j + 1] * y", "y"),
    "permute_tokens_descending": ("order = np.lexsort((flat_t, flat_e))", "order = np.lexsort((-flat_t, flat_e))"),
    "offsets_inclusive": ("offsets[1:] = np.cumsum(counts)", "offsets[1:] = np.cumsum(counts) - counts + 1"),
    "round_truncates": ("return np.rint(a / q) * q", "return np.trunc(a / q) * q"),
    "round_half_up": ("return np.rint(a / q) * q", "return np.floor(a / q + 0.5) * q"),
    "ylat_unrounded": ("y_lat = rnd(y_lat)", "y_lat = y_lat"),
    "h_unrounded": ("h = rnd(_relu2(z @ w_up.T))", "h = _relu2(z @ w_up.T)"),
    "down_uses_z": ("y = rnd(h @ w_down.T)", "y = rnd(h[:, :w_down.shape[0]] * 0 + z @ w_down[:, :z.shape[1]].T)"),
    "expert_weights_swapped": ("wu_bits, wd_bits = expert(e)", "wu_bits, wd_bits = expert((e + 1) % E)"),
    "decode_wrong_shift": ("astype(np.uint32) << 16", "astype(np.uint32) << 15"),
}


def load_mutant(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutant {name}: snippet not found in the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = load_mutant(name, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:   # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches the mutant {name}"
