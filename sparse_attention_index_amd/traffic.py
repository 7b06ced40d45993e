"""Algorithmic HBM bytes of the DSA decode step and of each kernel (for rooflines).

Per request, every context token's 132-byte index key (128 E4M3 values + fp32
scale; 68 bytes as MXFP4: 64 bytes of E2M1 pairs + 4 E8M0 block scales) is
read once for all of its rows. Per query row: the 2,048 selected
latent rows (576 E4M3 values + fp32 scale = 580 bytes) and the fp32 score of
every visible token, written by the scorer and read by the selection (the
pages count this round trip too: "TokenSpeed Kimi K3.1", section "Sparse
attention in Kimi K3.1 Pro", about 1 MB of scores at 128K tokens).
Small per-row terms (queries, head weights, selection, outputs) are included
where a kernel moves them.
"""

from __future__ import annotations

KEY_BYTES = 132
KEY_BYTES_MXFP4 = 68
LAT_ROW_BYTES = 580
SCORE_BYTES = 4
Q_IDX_BYTES = 32 * 128 * 2 + 32 * 2  # bf16 indexer query + bf16 head weights per row
Q_IDX_BYTES_FP8 = 32 * 128 + 4 + 32 * 2  # E4M3 indexer query + fp32 row scale + bf16 head weights
Q_MLA_BYTES = 16 * 576 * 2
OUT_BYTES = 16 * 512 * 2 + 16 * 4


def visible(ctx_lens, R):
    """Visible tokens of every row (position + 1)."""
    return [L - R + r + 1 for L in ctx_lens for r in range(R)]


def key_bytes(key_format="fp8"):
    return KEY_BYTES_MXFP4 if key_format == "mxfp4" else KEY_BYTES


def q_idx_bytes(q_fp8=False):
    return Q_IDX_BYTES_FP8 if q_fp8 else Q_IDX_BYTES


def scorer_bytes(ctx_lens, R, key_format="fp8", q_fp8=False):
    vis = visible(ctx_lens, R)
    return sum(ctx_lens) * key_bytes(key_format) + SCORE_BYTES * sum(vis) + len(vis) * q_idx_bytes(q_fp8)


def filter_scorer_bytes(ctx_lens, R, key_format="fp8", q_fp8=False):
    """The filtered scorer: keys once per request, the rows' queries and head
    weights; the (score, position) candidates it keeps (a few thousand per
    row, under 0.1% of the keys' bytes at 1M tokens) are not counted."""
    return sum(ctx_lens) * key_bytes(key_format) + len(visible(ctx_lens, R)) * q_idx_bytes(q_fp8)


def topk_bytes(ctx_lens, R, k):
    vis = visible(ctx_lens, R)
    return SCORE_BYTES * sum(vis) + 4 * k * len(vis)


def mla_bytes(ctx_lens, R, k):
    vis = visible(ctx_lens, R)
    return sum(min(k, v) * (LAT_ROW_BYTES + 4) for v in vis) + len(vis) * (Q_MLA_BYTES + OUT_BYTES)


def decode_step_bytes(ctx_lens, R, k, key_format="fp8", round_trip=True):
    """Keys once per request + per row: selected latents and, with
    round_trip, the fp32 score row written by the scorer and read by the
    selection (the stored-score path; the filtered path keeps no score row)."""
    vis = visible(ctx_lens, R)
    rt = 2 * SCORE_BYTES if round_trip else 0
    return sum(ctx_lens) * key_bytes(key_format) + sum(min(k, v) * LAT_ROW_BYTES + rt * v for v in vis)


def scorer_flops(ctx_lens, R, heads=32, dim=128):
    return 2 * heads * dim * sum(visible(ctx_lens, R))
