"""Parity checks of GPU results against the oracle, with the tolerances of the method.

* Scores: relative 1e-3, |g - r| <= 1e-3 * max(|r|, 1e-6 * max_row |r|); the
  floor only matters where the exact score is (near) zero.
* Selection on identical fp32 scores: exact set equality (integer work).
* Selection against the oracle's float64 scores: the sets have equal size
  and every position in their symmetric difference scores within 1e-3
  (relative) of the oracle's k-th largest score.
* Attention: per (row, head), max_v |g - r| <= 1e-2 * max_v |r|; lse within
  1e-4 * max(1, |r|).
"""

from __future__ import annotations

import numpy as np

import oracle

SCORE_RTOL = 1e-3
TOPK_BAND = 1e-3
OUT_RTOL = 1e-2
LSE_TOL = 1e-4


def check_scores(g, r, what=""):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU scores at {np.where(~np.isfinite(g))[0][:8]}"
    floor = 1e-6 * (np.abs(r).max() if r.size else 0.0)
    tol = SCORE_RTOL * np.maximum(np.abs(r), floor)
    bad = np.abs(g - r) > tol
    assert not bad.any(), (
        f"{what}: {bad.sum()} scores off, worst at {np.argmax(np.abs(g - r) - tol)}: "
        f"gpu {g[bad][:4]} oracle {r[bad][:4]}"
    )


def sel_set(row_idx, n_visible):
    row_idx = np.asarray(row_idx)
    valid = row_idx[row_idx >= 0]
    assert valid.size == np.unique(valid).size, "duplicate positions in a selection"
    assert np.all(valid < n_visible), "a selected position is not visible to the row"
    return set(valid.tolist())


def check_topk_exact(gpu_row_idx, scores32, k, what=""):
    n = scores32.size
    got = sel_set(gpu_row_idx, n)
    want = set(oracle.topk_positions(np.asarray(scores32, np.float64), k).tolist())
    assert len(got) == min(k, n), f"{what}: selected {len(got)} of {min(k, n)}"
    pad = np.asarray(gpu_row_idx)[min(k, n):]
    assert np.all(pad == -1), f"{what}: padding is not -1"
    assert got == want, f"{what}: {len(got ^ want)} positions differ"


def check_topk_band(gpu_row_idx, oracle_scores, k, what=""):
    s = np.asarray(oracle_scores, np.float64)
    n = s.size
    got = sel_set(gpu_row_idx, n)
    ref = oracle.topk_positions(s, k)
    want = set(ref.tolist())
    assert len(got) == len(want) == min(k, n), f"{what}: {len(got)} vs {len(want)}"
    diff = np.array(sorted(got ^ want), dtype=np.int64)
    if diff.size:
        tau = s[ref[-1]]
        off = np.abs(s[diff] - tau)
        assert np.all(off <= TOPK_BAND * abs(tau)), (
            f"{what}: {diff.size} positions differ, farthest {off.max()} from tau {tau}"
        )
    return diff.size


def check_attention(out_g, lse_g, out_r, lse_r, what=""):
    g = np.asarray(out_g, np.float64)
    r = np.asarray(out_r, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    scale = np.abs(r).max(axis=-1)
    err = np.abs(g - r).max(axis=-1)
    ok = err <= OUT_RTOL * scale
    ok |= (scale == 0) & (err == 0)
    assert ok.all(), f"{what}: worst relative error {(err / np.maximum(scale, 1e-30)).max():.3g}"
    if lse_g is not None:
        lg, lr = np.asarray(lse_g, np.float64), np.asarray(lse_r, np.float64)
        both_inf = np.isneginf(lg) & np.isneginf(lr)
        with np.errstate(invalid="ignore"):
            d = np.where(both_inf, 0.0, np.abs(lg - lr))
        assert np.all(d <= LSE_TOL * np.maximum(1.0, np.abs(lr))), f"{what}: lse off by {d.max():.3g}"
