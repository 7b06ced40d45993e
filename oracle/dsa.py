"""The DSA hot path written out as its plain definition, in float64.

Steps follow "TokenSpeed Kimi K3.1", section "Integrating sparse attention
with the K3 stack": Score (the indexer's 32 heads score every cached index
key), Select (the 2,048 highest-scoring positions per query row), Attend
(MLA over only those latent rows). The cache is paged in 64-token blocks and
both planes (index keys and latents) share one block table.

Readings where the pages are silent (each is listed in the design doc):
* a row at position p sees tokens 0..p, its own token included (the Write
  step runs before Score, so the row's key is already cached);
* the score of token s is sum_h w_h * ReLU(q_h . khat_s) with khat_s the
  dequantised key (E4M3 value times the token's fp32 scale, or for MXFP4
  keys each E2M1 value times its block's power of two); no other constant
  is applied;
* selection keeps min(k, visible) positions, ranked by score descending,
  ties broken by the lower position;
* attention uses softmax over scale * q . chat_s on all 576 dims, values are
  the first 512 dims of chat_s, lse is the natural-log log-sum-exp.
"""

from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode
from .mxfp4 import mxfp4_decode

BLOCK = 64


def gather_tokens(plane, block_table_row, positions):
    """Rows of a paged cache plane for logical token positions of one request.

    plane: [num_blocks, 64, ...]; block_table_row: [max_blocks] page ids.
    """
    positions = np.asarray(positions, dtype=np.int64)
    table = np.asarray(block_table_row, dtype=np.int64)
    pages = table[positions // BLOCK]
    assert np.all(pages >= 0), "position outside the request's pages"
    return np.asarray(plane)[pages, positions % BLOCK]


def dequant(codes, scale):
    """E4M3 codes [n, d] times a per-token scale [n] -> float64 [n, d]."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def index_scores(q, w, keys_hat):
    """Indexer score of each key: sum_h w[h] * relu(q[h] . keys_hat[s]).

    q: [H, D] float64, w: [H], keys_hat: [n, D] -> [n] float64.
    """
    dots = np.asarray(keys_hat, np.float64) @ np.asarray(q, np.float64).T  # [n, H]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def topk_positions(scores, k):
    """Brute-force selection by a full sort: the min(k, n) largest scores,
    ties broken by the lower position. Returned in rank order."""
    s = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((np.arange(s.size), -s))
    return order[: min(k, s.size)]


def attend(q, rows_hat, sm_scale, dv=512):
    """Exact softmax attention of q [H, 576] over latent rows [n, 576].

    Returns (out [H, dv], lse [H]). With n == 0 the output is 0 and lse -inf.
    """
    q = np.asarray(q, np.float64)
    rows_hat = np.asarray(rows_hat, np.float64)
    H = q.shape[0]
    if rows_hat.shape[0] == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    logits = sm_scale * (q @ rows_hat.T)  # [H, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ rows_hat[:, :dv]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def _np(t):
    """torch tensor (any dtype, any device) or array -> numpy (bf16 via float32, exact)."""
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.bfloat16":
            t = t.float()
        return t.numpy()
    return np.asarray(t)


def _query_rows(case):
    """Indexer queries as float64 [rows, 32, 128] (dequantising FP8 query rows)."""
    if case.q_idx_scale is not None:
        return e4m3_decode(_np(case.q_idx)) * _np(case.q_idx_scale).astype(np.float64)[:, None, None]
    return _np(case.q_idx).astype(np.float64)


def row_scores(case, row, positions=None, q_rows=None):
    """Scores of one query row over `positions` (default: all it sees)."""
    B, R = case.B, case.R
    b = row // R
    pos = int(_np(case.ctx_len)[b]) - R + row % R
    if positions is None:
        positions = np.arange(pos + 1)
    positions = np.asarray(positions, dtype=np.int64)
    assert positions.size == 0 or positions.max() <= pos, "score requested for an unseen token"
    table = _np(case.block_table)[b]
    if getattr(case, "key_format", "fp8") == "mxfp4":
        keys_hat = mxfp4_decode(gather_tokens(_np(case.key_fp4), table, positions),
                                gather_tokens(_np(case.key_e8m0), table, positions))
    else:
        keys_hat = dequant(gather_tokens(_np(case.key_fp8), table, positions),
                           gather_tokens(_np(case.key_scale), table, positions))
    q = (q_rows if q_rows is not None else _query_rows(case))[row]
    return index_scores(q, _np(case.w)[row].astype(np.float64), keys_hat)


def dense_attend_row(case, row, positions):
    """Attention of one row's MLA query over the latent rows at `positions`
    (entries < 0 are ignored)."""
    b = row // case.R
    positions = np.asarray(positions, dtype=np.int64)
    positions = positions[positions >= 0]
    table = _np(case.block_table)[b]
    rows_hat = dequant(gather_tokens(_np(case.lat_fp8), table, positions),
                       gather_tokens(_np(case.lat_scale), table, positions))
    return attend(_np(case.q_mla)[row].astype(np.float64), rows_hat, case.sm_scale)


def dsa_rows(case, rows=None, idx=None, k=None):
    """Run Score -> Select -> Attend for the given query rows.

    If idx ([rows_total, k] positions, -1 padded) is given, Attend uses those
    positions instead of the oracle's own selection (used to check the
    attention stage on another implementation's selection).
    Returns dict row -> {"scores", "sel", "out", "lse"}.
    """
    k = case.topk if k is None else k
    rows = range(case.rows) if rows is None else rows
    q_rows = _query_rows(case)
    res = {}
    for row in rows:
        s = row_scores(case, row, q_rows=q_rows)
        sel = topk_positions(s, k)
        use = sel if idx is None else np.asarray(_np(idx)[row], dtype=np.int64)
        out, lse = dense_attend_row(case, row, use)
        res[row] = {"scores": s, "sel": sel, "out": out, "lse": lse}
    return res
