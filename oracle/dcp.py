"""Exact top-k merge and LSE combine under decode context parallelism,
simulated on one device -- TEST INFRASTRUCTURE ONLY (see the package docstring).

The steps follow "Kimi K3.1 Pro: Day-0 Inference and RL Support with SGLang and Miles", section "Decode:
DSA with decode context parallelism", and "vLLM Day-0 Support for Kimi K3.1
Pro", section "An exact top-k merge with about 10x less traffic":
1. token p lives on shard p mod W; each shard scores only its tokens;
2. each shard takes its local top-k (no global winner is lost: a token in
   the global top-k is in the top-k of its own shard);
3. each shard sends its best C candidates (C = 1.5 k / W: 384 for k = 2048,
   W = 8); every shard sees the same W x C candidates;
4. the cutoff is the k-th best of those candidates;
5. a shard whose C candidates all beat the cutoff may hold more winners
   than it sent, so its full local top-k joins the candidates (one whose
   C-th candidate is the cutoff or below cannot: everything it kept back
   ranks below the cutoff);
6. the k best of the resulting pool are the global top-k, the same set a
   single device selects;
7. each shard attends to the winners it owns, and the partial outputs are
   combined by their log-sum-exp ("TokenSpeed Kimi K3.1", section
   "Sharding long contexts with decode context parallelism", steps 3-4).

Readings: candidates and winners are ranked by score, ties broken by the
lower position (the same total order as the single-device selection, so
"falls below" is strict in that order); a shard with fewer than C tokens
sends them all and never needs to resend; with fewer than k candidates in
all there is no cutoff and every shard that sent C candidates resends.
"""

import numpy as np

from .dsa import attend, topk_positions


def _rank_key(scores, positions):
    """Sort key of the total order: higher score first, then lower position."""
    return np.lexsort((positions, -scores))


def shard_positions(n, W, w):
    """Positions 0..n-1 that shard w holds (p mod W == w), ascending."""
    return np.arange(w, n, W, dtype=np.int64)


def local_topk(scores, W, w, k):
    """Shard w's best min(k, |shard|) positions, best first."""
    pos = shard_positions(len(scores), W, w)
    order = topk_positions(np.asarray(scores, np.float64)[pos], k)
    return pos[order]


def _better(scores, a, b):
    """Position a ranks strictly above position b in the total order."""
    return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)


def dcp_select(scores, W, k, C=None):
    """The exact merged top-k of one row's scores over W shards.

    Returns (selected positions best first, resend flags [W], cutoff
    position or -1 when there is no cutoff)."""
    s = np.asarray(scores, np.float64)
    C = int(1.5 * k / W) if C is None else C
    local = [local_topk(s, W, w, k) for w in range(W)]
    sent = [lt[:C] for lt in local]
    cand = np.concatenate(sent)
    if cand.size >= k:
        order = _rank_key(s[cand], cand)
        cutoff = int(cand[order[k - 1]])
    else:
        cutoff = -1
    resend = np.zeros(W, dtype=bool)
    for w in range(W):
        if len(sent[w]) < C:  # sent everything it holds
            continue
        last = int(sent[w][C - 1])
        resend[w] = cutoff < 0 or _better(s, last, cutoff)  # all C sent beat the cutoff
    pool = np.unique(np.concatenate([local[w] if resend[w] else sent[w] for w in range(W)]))
    order = _rank_key(s[pool], pool)
    return pool[order[: min(k, pool.size)]], resend, cutoff


def shard_attend(q, rows_hat_by_pos, positions, W, w, sm_scale):
    """Partial attention of shard w over the selected positions it owns."""
    positions = np.asarray(positions, np.int64)
    own = positions[positions % W == w]
    return attend(q, rows_hat_by_pos(own), sm_scale)


def lse_combine(outs, lses):
    """Combine partial outputs [W][H, dv] with their log-sum-exps [W][H]:
    out = sum_w exp(lse_w - L) out_w with L = log sum_w exp(lse_w)."""
    lses = np.asarray(lses, np.float64)  # [W, H]
    outs = np.asarray(outs, np.float64)  # [W, H, dv]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    wts = np.where(np.isfinite(lses), np.exp(lses - msafe), 0.0)  # [W, H]
    tot = wts.sum(axis=0)
    L = np.where(finite, msafe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    out = np.where(finite[:, None], (wts[:, :, None] * outs).sum(axis=0) / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return out, L
