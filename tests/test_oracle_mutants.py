"""The oracle's pins catch plausible mistakes.

Each mutant replaces one oracle function by a version with a typical slip (a
dropped term, a wrong sign, a swapped index, an off-by-one) and runs the pins
against it; at least one pin must fail for every mutant. Mistakes are planted
only in the CPU oracle, never in GPU code.
"""

import numpy as np
import pytest

import oracle
import oracle.dsa as odsa
from oracle import fp8 as ofp8
from tests import test_oracle_pins as pins


def _scores_no_relu(q, w, k):
    return (np.asarray(k) @ np.asarray(q).T) @ np.asarray(w)


def _scores_no_weights(q, w, k):
    return np.maximum(np.asarray(k) @ np.asarray(q).T, 0.0).sum(axis=1)


def _scores_abs(q, w, k):
    return np.abs(np.asarray(k) @ np.asarray(q).T) @ np.asarray(w)


def _scores_relu_after_sum(q, w, k):
    return np.maximum((np.asarray(k) @ np.asarray(q).T) @ np.asarray(w), 0.0)


def _topk_high_index_ties(s, k):
    s = np.asarray(s, np.float64)
    order = np.lexsort((-np.arange(s.size), -s))
    return order[: min(k, s.size)]


def _topk_short(s, k):
    return _orig["topk_positions"](s, k)[:-1]


def _attend_wrong_slice(q, rows, sm, dv=512):
    # values taken from the last 512 latent dims instead of the first 512
    q, rows = np.asarray(q, np.float64), np.asarray(rows, np.float64)
    if rows.shape[0] == 0:
        return _orig["attend"](q, rows, sm, dv)
    logits = sm * (q @ rows.T)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ rows[:, 64 : 64 + dv]) / l, (m + np.log(l))[:, 0]


def _attend_no_scale(q, rows, sm, dv=512):
    return _orig["attend"](q, rows, 1.0, dv)


def _attend_lse_log2(q, rows, sm, dv=512):
    out, lse = _orig["attend"](q, rows, sm, dv)
    return out, lse / np.log(2.0)


def _dequant_no_scale(codes, scale):
    return ofp8.e4m3_decode(codes) * 1.0


def _gather_off_by_one(plane, table_row, positions):
    positions = np.asarray(positions, dtype=np.int64)
    table = np.asarray(table_row, dtype=np.int64)
    p = np.minimum(positions + 1, table[table >= 0].size * 64 - 1)
    return np.asarray(plane)[table[p // 64], p % 64]


_orig = {
    "index_scores": odsa.index_scores,
    "topk_positions": odsa.topk_positions,
    "attend": odsa.attend,
    "dequant": odsa.dequant,
    "gather_tokens": odsa.gather_tokens,
}

MUTANTS = {
    "score_without_relu": ("index_scores", _scores_no_relu),
    "score_without_head_weights": ("index_scores", _scores_no_weights),
    "score_abs_instead_of_relu": ("index_scores", _scores_abs),
    "score_relu_after_head_sum": ("index_scores", _scores_relu_after_sum),
    "topk_ties_to_higher_position": ("topk_positions", _topk_high_index_ties),
    "topk_one_short": ("topk_positions", _topk_short),
    "attend_values_from_wrong_dims": ("attend", _attend_wrong_slice),
    "attend_without_softmax_scale": ("attend", _attend_no_scale),
    "attend_lse_in_log2": ("attend", _attend_lse_log2),
    "dequant_drops_token_scale": ("dequant", _dequant_no_scale),
    "gather_off_by_one_token": ("gather_tokens", _gather_off_by_one),
}

PIN_TESTS = [
    (pins.test_scores_relu_difference_identity, ()),
    (pins.test_scores_relu_sum_identity, ()),
    (pins.test_scores_hand_worked_example, ()),
    (pins.test_scores_homogeneous_and_linear_in_weights, ()),
    (pins.test_topk_matches_heapq_with_ties, (5000, 2048)),
    (pins.test_topk_matches_heapq_with_ties, (3000, 64)),
    (pins.test_topk_planted_winners, ()),
    (pins.test_attend_matches_torch_sdpa, ()),
    (pins.test_attend_single_row_and_zero_query, ()),
    (pins.test_short_context_sparse_equals_dense, ()),
    (pins.test_causal_rows_never_see_later_tokens, ()),
    (pins.test_fp8_query_rows_dequantise_with_their_scale, ()),
    (pins.test_counted_bytes_of_an_oracle_run_match_the_closed_form, ()),
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_the_mutant(mutant, monkeypatch):
    fname, fn = MUTANTS[mutant]
    monkeypatch.setattr(odsa, fname, fn)
    if hasattr(oracle, fname):
        monkeypatch.setattr(oracle, fname, fn)
    caught = []
    for test, args in PIN_TESTS:
        try:
            test(*args)
        except (AssertionError, IndexError, ValueError):
            caught.append(test.__name__)
    assert caught, f"no pin caught mutant {mutant}"
