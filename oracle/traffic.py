"""Bytes a decode step reads per layer, dense MLA versus DSA.

Byte model of "TokenSpeed Kimi K3.1", section "Sparse attention in Kimi K3.1
Pro": dense MLA reads every earlier token's FP8 latent row; DSA reads every
earlier token's 132-byte index key, then the latent rows of the 2,048 selected
tokens, plus the index scores (fp32, written once and read once: 8 bytes per
row per token). The index keys are read once for all of a request's
verification rows. "vLLM Day-0 Support for Kimi K3.1 Pro", section "Sparse
attention cuts long-context decode bandwidth", gives the long-context limit of
the ratio as about 23%.
"""

import numpy as np

KEY_BYTES = 132  # 128 FP8 values + fp32 scale
LAT_BYTES = 576  # 576 FP8 values (the pages' count, without a scale)
SCORE_BYTES = 8  # fp32 score written once and read once


def dense_mla_bytes(n_ctx, lat_bytes=LAT_BYTES):
    """Latent bytes dense MLA reads for one request (rows share the read)."""
    return n_ctx * lat_bytes


def dsa_bytes(n_ctx, rows=1, k=2048, key_bytes=KEY_BYTES, lat_bytes=LAT_BYTES,
              score_bytes=SCORE_BYTES):
    """Bytes DSA reads for one request with `rows` query rows."""
    return n_ctx * key_bytes + rows * (min(k, n_ctx) * lat_bytes + n_ctx * score_bytes)


def counted_bytes(case, results, key_bytes=KEY_BYTES, lat_bytes=LAT_BYTES,
                  score_bytes=SCORE_BYTES):
    """Bytes the oracle's own run touched, counted from what it gathered.

    results: output of dsa_rows for every row of `case`. Keys: each distinct
    (request, token) scored counts once. Latents: each selected (row, token).
    Scores: one per (row, token) scored.
    """
    keys = {}
    lat = 0
    sc = 0
    for row, r in results.items():
        b = row // case.R
        n = r["scores"].size
        keys[b] = max(keys.get(b, 0), n)
        sc += n
        lat += int(np.count_nonzero(np.asarray(r["sel"]) >= 0))
    return sum(keys.values()) * key_bytes + lat * lat_bytes + sc * score_bytes
