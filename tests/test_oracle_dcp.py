"""Pins of the DCP merge oracle: the merged selection must equal the
single-device top-k (the pages' claim, checked against the brute-force sort
that the top-k pins fix), on random, tied, short and adversarial rows; the
resend rule must fire exactly where a shard holds more winners than it sent;
the LSE combine of any partition must equal attention over the union. Plus
mutants these pins catch.
"""

import numpy as np
import pytest

import oracle
import oracle.dcp as odcp

RNG = np.random.default_rng(20260303)


def _rows():
    out = []
    for n in (5, 700, 2047, 2048, 2049, 2060, 9000, 30000):
        out.append(RNG.standard_normal(n))
    out.append(RNG.integers(0, 4, size=12000).astype(np.float64))  # heavy ties
    out.append(np.zeros(5000))  # all tied: lowest positions win
    x = RNG.standard_normal(20000)
    x[0::8] += 10.0  # every winner on shard 0 (W = 8), and on shards 0/4 for W = 4 ...
    out.append(x)
    y = RNG.standard_normal(20000)
    y[3:3000:8] += 10.0  # 375 boosted tokens on shard 3: fewer than C, no resend needed
    out.append(y)
    return out


@pytest.mark.parametrize("W", [2, 4, 8])
def test_merged_selection_equals_single_device_topk(W):
    for s in _rows():
        sel, _, _ = oracle.dcp_select(s, W, 2048)
        want = oracle.topk_positions(s, 2048)
        assert np.array_equal(sel, want), (W, s.size)


def test_default_candidate_count_is_the_pages_384():
    s = RNG.standard_normal(40000)
    _, _, _ = oracle.dcp_select(s, 8, 2048)
    assert int(1.5 * 2048 / 8) == 384
    # with C = 384 explicitly the result is the same
    assert np.array_equal(oracle.dcp_select(s, 8, 2048)[0], oracle.dcp_select(s, 8, 2048, C=384)[0])


def test_global_winners_are_in_their_shards_local_topk():
    s = RNG.standard_normal(25000)
    win = set(oracle.topk_positions(s, 2048).tolist())
    for w in range(8):
        local = set(oracle.local_topk(s, 8, w, 2048).tolist())
        assert {p for p in win if p % 8 == w} <= local


def test_resend_fires_only_for_a_shard_holding_too_many_winners():
    s = RNG.standard_normal(20000)
    s[0::8] += 10.0  # shard 0 holds all 2,048 winners
    _, resend, _ = oracle.dcp_select(s, 8, 2048)
    assert resend.tolist() == [True] + [False] * 7
    _, resend, _ = oracle.dcp_select(RNG.standard_normal(20000), 8, 2048)
    assert not resend.any()
    # a shard with fewer than C tokens sends them all and never resends
    _, resend, cutoff = oracle.dcp_select(RNG.standard_normal(2000), 8, 2048)
    assert cutoff == -1 and not resend.any()


def test_resend_matches_its_definition_on_random_rows():
    for _ in range(20):
        s = RNG.standard_normal(RNG.integers(3000, 20000))
        s[RNG.integers(0, 8)::8] += RNG.uniform(0, 3)
        sel, resend, cutoff = oracle.dcp_select(s, 8, 2048)
        for w in range(8):
            kept = oracle.local_topk(s, 8, w, 2048)
            # a shard holds more winners than its 384 sent iff it resent
            n_win = len(set(kept.tolist()) & set(sel.tolist()))
            if n_win > 384:
                assert resend[w]


def test_lse_combine_equals_attention_over_the_union():
    H, D = 4, 576
    for n, W in ((300, 8), (50, 4), (7, 8), (2048, 2)):
        q = RNG.standard_normal((H, D))
        rows = RNG.standard_normal((n, D)) * 0.3
        owner = RNG.integers(0, W, size=n)
        outs, lses = [], []
        for w in range(W):
            o, l = oracle.attend(q, rows[owner == w], 1 / 24)
            outs.append(o)
            lses.append(l)
        out, lse = oracle.lse_combine(outs, lses)
        ro, rl = oracle.attend(q, rows, 1 / 24)
        assert np.allclose(out, ro, rtol=1e-10, atol=1e-12) and np.allclose(lse, rl, rtol=1e-12)


def test_shard_attend_owns_positions_mod_w_and_combines_to_attention():
    """Shard w attends over exactly the selected positions p with p mod W == w
    (token striping of decode context parallelism), and the LSE combine of
    the W shards' partials is attention over the whole selection."""
    H, D = 4, 576
    table = RNG.standard_normal((6000, D)) * 0.3
    for n, W in ((300, 8), (41, 3), (2048, 2), (5, 8)):
        q = RNG.standard_normal((H, D))
        positions = RNG.choice(6000, size=n, replace=False)
        asked = []

        def rows_hat_by_pos(p):
            asked.append(np.asarray(p, np.int64).copy())
            return table[np.asarray(p, np.int64)]

        outs, lses = [], []
        for w in range(W):
            o, l = oracle.shard_attend(q, rows_hat_by_pos, positions, W, w, 1 / 24)
            outs.append(o)
            lses.append(l)
        for w in range(W):
            want = sorted(p for p in positions.tolist() if p % W == w)
            assert sorted(asked[w].tolist()) == want, (n, W, w)
        out, lse = oracle.lse_combine(outs, lses)
        ro, rl = oracle.attend(q, table[positions], 1 / 24)
        assert np.allclose(out, ro, rtol=1e-10, atol=1e-12) and np.allclose(lse, rl, rtol=1e-12)


def test_lse_combine_of_nothing_is_empty_attention():
    out, lse = oracle.lse_combine(np.zeros((3, 2, 512)), np.full((3, 2), -np.inf))
    assert not out.any() and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- mutants

_ORIG = {n: getattr(odcp, n) for n in ("dcp_select", "lse_combine", "shard_attend")}


def _select_cutoff_off_by_one(scores, W, k, C=None):
    return _ORIG["dcp_select"](scores, W, k - 1 if k > 1 else k, C)  # selects one too few, cutoff one early


def _select_no_resend(scores, W, k, C=None):
    s = np.asarray(scores, np.float64)
    C = int(1.5 * k / W) if C is None else C
    sent = np.concatenate([odcp.local_topk(s, W, w, k)[:C] for w in range(W)])
    order = np.lexsort((sent, -s[sent]))
    return sent[order[:k]], np.zeros(W, bool), -1


def _select_ties_by_higher_position(scores, W, k, C=None):
    s = np.asarray(scores, np.float64)
    sel, resend, cut = _ORIG["dcp_select"](s, W, k, C)
    order = np.lexsort((-sel, -s[sel]))
    return sel[order], resend, cut


def _combine_without_weights(outs, lses):
    _, L = _ORIG["lse_combine"](outs, lses)
    return np.asarray(outs, np.float64).mean(axis=0), L


def _shard_attend_shifted_owner(q, rows_hat_by_pos, positions, W, w, sm_scale):
    return _ORIG["shard_attend"](q, rows_hat_by_pos, np.asarray(positions, np.int64) + 1, W, w, sm_scale)


def _shard_attend_every_position(q, rows_hat_by_pos, positions, W, w, sm_scale):
    return odcp.attend(q, rows_hat_by_pos(np.asarray(positions, np.int64)), sm_scale)


MUTANTS = {
    "cutoff_off_by_one": ("dcp_select", _select_cutoff_off_by_one),
    "never_resends": ("dcp_select", _select_no_resend),
    "ties_to_higher_position": ("dcp_select", _select_ties_by_higher_position),
    "combine_unweighted": ("lse_combine", _combine_without_weights),
    "shard_owner_shifted": ("shard_attend", _shard_attend_shifted_owner),
    "shard_takes_every_position": ("shard_attend", _shard_attend_every_position),
}

PIN_TESTS = [
    lambda: test_merged_selection_equals_single_device_topk(8),
    test_resend_fires_only_for_a_shard_holding_too_many_winners,
    test_lse_combine_equals_attention_over_the_union,
    test_shard_attend_owns_positions_mod_w_and_combines_to_attention,
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_the_dcp_mutant(mutant, monkeypatch):
    fname, fn = MUTANTS[mutant]
    monkeypatch.setattr(odcp, fname, fn)
    monkeypatch.setattr(oracle, fname, fn)
    caught = 0
    for test in PIN_TESTS:
        try:
            test()
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught, f"no pin caught mutant {mutant}"
