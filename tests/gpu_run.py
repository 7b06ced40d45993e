"""Drive the C-ABI entry points on a seeded case and bring results to the host.

Used by the GPU parity tests only. Buffers come from torch (device memory);
every computation happens in libdsa.
"""

from __future__ import annotations

import math

import torch

import sparse_attention_index_amd as dsa


def ld_for(case) -> int:
    return int(math.ceil(case.max_ctx / 64) * 64)


def gpu_scores(case, sentinel=float("nan")):
    """fp32 [rows, ld] scores; entries the kernel must not write keep `sentinel`."""
    ld = ld_for(case)
    scores = torch.full((case.rows, ld), sentinel, dtype=torch.float32, device="cuda")
    dsa.dsa_index_score(dsa.Batch.of(case), dsa.Cache.of(case), case.q_idx, case.w, scores,
                        q_scale=case.q_idx_scale)
    return scores


def row_len_of(case) -> torch.Tensor:
    return (case.positions() + 1).to(torch.int32).cuda()


def gpu_topk(scores, row_len, k):
    rows, ld = scores.shape
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, rows, ld, k))
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(scores, row_len, k, idx, ws)
    return idx


def gpu_mla(case, idx, split=True, with_lse=True):
    rows, k = idx.shape
    kind = dsa.DSA_WS_MLA_DECODE if split else dsa.DSA_WS_MLA_PREFILL
    nbytes = dsa.dsa_workspace_size(kind, rows, 0, k)
    ws = dsa.workspace(nbytes) if nbytes else None
    out = torch.full((rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    fn = dsa.dsa_sparse_mla_decode if split else dsa.dsa_sparse_mla_prefill
    fn(dsa.Batch.of(case), dsa.Cache.of(case), case.q_mla, idx, case.sm_scale, out, lse, ws)
    return out, lse


def gpu_decode(case, k=None, threshold=None):
    """The fused decode; with `threshold` (fp32 [rows]) through dsa_decode_thresholded."""
    k = case.topk if k is None else k
    rows = case.rows
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, rows, case.max_ctx, k))
    ws.fill_(0xA5)  # stale workspace contents must not matter
    out = torch.full((rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_decode(dsa.Batch.of(case), dsa.Cache.of(case), case.q_idx, case.w, case.q_mla, k, case.sm_scale,
                   out, lse, idx, ws, threshold=threshold, q_scale=case.q_idx_scale)
    return out, lse, idx
