"""GPU parity at the full sizes of the named workloads, in the launch
configuration the benchmark times.

Decode workloads run the fused dsa_decode over the whole batch (the
benchmark's step), then the stage-wise entry points on the same inputs:
* the fused and the stage-wise selections are the same set on every row, and
  the outputs agree;
* the selection of every row equals the oracle's selection applied to the
  GPU's own fp32 scores (exact integer work, decided in fp32 on both sides);
* on sampled rows (first, last and a seeded pick) the scores match the
  float64 oracle, no score past the row's position is written, the selection
  lies within the tolerance band of the oracle's scores, and the attention
  output matches the oracle run on the GPU's selection.
The prefill chunk runs score -> top-k -> sparse MLA prefill over all 4,096
rows and checks sampled rows the same way.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import gpu_decode, gpu_mla, gpu_scores, gpu_topk, row_len_of
from tests.parity import check_attention, check_scores, check_topk_band, check_topk_exact
from workloads import case_config, make_case, structure_kwargs

pytestmark = pytest.mark.gpu

DECODE = ["decode_1x1_8k", "decode_16x4_32k", "decode_16x8_32k", "decode_16x4_ragged_128k_256k",
          "decode_4x4_1m_planted", "decode_4x4_1m_mxfp4", "decode_4x4_1m_recent", "decode_16x4_256k_1m",
          "decode_4x4_1m_fp8q"]


def _make(name):
    cfg = case_config(name)
    kw = structure_kwargs(cfg)
    print(f"\n[fullsize] {name} B={cfg['B']} R={cfg['R']} lengths[0:4]={cfg['lengths'][:4]}", flush=True)
    return make_case(cfg["B"], cfg["R"], cfg["lengths"], seed=cfg["seed"], device="cuda", name=name, **kw)


def _sample_rows(rows, n_extra=1, seed=0):
    pick = {0, rows - 1}
    rng = np.random.default_rng(seed)
    pick.update(rng.integers(0, rows, size=n_extra).tolist())
    return sorted(pick)


def _visible(case):
    return (case.positions() + 1).numpy()


@pytest.mark.parametrize("name", DECODE)
def test_decode_workload_full_size(gpu, name):
    case = _make(name)
    out, lse, idx = gpu_decode(case)
    scores = gpu_scores(case)
    s_idx = gpu_topk(scores, row_len_of(case), case.topk)
    s_out, s_lse = gpu_mla(case, s_idx)
    torch.cuda.synchronize()
    print("[fullsize] GPU done", flush=True)

    vis = _visible(case)
    idx_h, s_idx_h = idx.cpu().numpy(), s_idx.cpu().numpy()
    scores_h = scores.cpu().numpy()
    out_h, lse_h = out.float().cpu().numpy(), lse.cpu().numpy()
    s_out_h, s_lse_h = s_out.float().cpu().numpy(), s_lse.cpu().numpy()
    for row in range(case.rows):
        n = int(vis[row])
        assert set(idx_h[row].tolist()) == set(s_idx_h[row].tolist()), f"{name} row {row}: fused vs staged"
        check_topk_exact(idx_h[row], scores_h[row, :n], case.topk, f"{name} row {row}")
        assert np.all(np.isnan(scores_h[row, n:])), f"{name} row {row}: score written past the position"
    # same selection, same kernels: the staged outputs agree with the fused ones
    check_attention(s_out_h, s_lse_h, out_h, lse_h, f"{name} staged vs fused")

    if name.endswith("_recent"):
        # the workload's structure: most of every row's selection lies in its last 32K positions
        L = case.ctx_len.cpu().numpy()
        for row in range(case.rows):
            frac = np.mean(idx_h[row] >= int(L[row // case.R]) - 32768)
            assert frac >= 0.75, f"{name} row {row}: only {frac:.2f} of the selection in the recency window"
    host = case.to("cpu")
    rows = _sample_rows(case.rows, n_extra=1 if case.rows < 64 else 6, seed=7)
    res = oracle.dsa_rows(host, rows=rows, idx=idx_h)
    for row in rows:
        n = int(vis[row])
        check_scores(scores_h[row, :n], res[row]["scores"], f"{name} row {row}")
        check_topk_band(idx_h[row], res[row]["scores"], case.topk, f"{name} row {row}")
        check_attention(out_h[row], lse_h[row], res[row]["out"], res[row]["lse"], f"{name} row {row}")
        print(f"[fullsize] {name} row {row} ok", flush=True)


def test_prefill_chunk_full_size(gpu):
    name = "prefill_4096_on_128k"
    case = _make(name)
    scores = gpu_scores(case)
    idx = gpu_topk(scores, row_len_of(case), case.topk)
    out, lse = gpu_mla(case, idx, split=False)
    torch.cuda.synchronize()
    print("[fullsize] GPU done", flush=True)

    vis = _visible(case)
    rows = _sample_rows(case.rows, n_extra=2, seed=11)
    exact_rows = sorted(set(rows) | set(range(0, case.rows, 128)))
    idx_h = idx.cpu().numpy()
    for row in exact_rows:
        n = int(vis[row])
        srow = scores[row].cpu().numpy()
        check_topk_exact(idx_h[row], srow[:n], case.topk, f"{name} row {row}")
        assert np.all(np.isnan(srow[n:])), f"{name} row {row}: score written past the position"

    host = case.to("cpu")
    res = oracle.dsa_rows(host, rows=rows, idx=idx_h)
    out_h, lse_h = out.float().cpu().numpy(), lse.cpu().numpy()
    for row in rows:
        n = int(vis[row])
        check_scores(scores[row, :n].cpu().numpy(), res[row]["scores"], f"{name} row {row}")
        check_topk_band(idx_h[row], res[row]["scores"], case.topk, f"{name} row {row}")
        check_attention(out_h[row], lse_h[row], res[row]["out"], res[row]["lse"], f"{name} row {row}")
        print(f"[fullsize] {name} row {row} ok", flush=True)
