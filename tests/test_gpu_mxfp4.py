"""GPU parity of the scorer on MXFP4 index keys, and of the fused decode
built on it, against the oracle (which decodes the E2M1 codes and E8M0 block
scales exactly). The same tolerances as for FP8 keys apply: scores 1e-3
relative; selections exact on the GPU's own scores and within the tolerance
band of the oracle's; attention 1e-2.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_run import gpu_decode, gpu_scores, gpu_topk, row_len_of
from tests.parity import check_attention, check_scores, check_topk_band, check_topk_exact
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = {
    "f4_1x4_3k": dict(B=1, R=4, lengths=[3000], seed=501),
    "f4_2x3_perm": dict(B=2, R=3, lengths=[5001, 700], seed=502, permute_blocks=True),
    "f4_1x8": dict(B=1, R=8, lengths=[2500], seed=503),
    "f4_2x1_tiny": dict(B=2, R=1, lengths=[130, 64], seed=504),
    "f4_fp8q_1x64": dict(B=1, R=64, lengths=[2048 + 64], seed=505, fp8_query=True),
    "f4_fp8q_2x7": dict(B=2, R=7, lengths=[3333, 5000], seed=506, fp8_query=True, permute_blocks=True),
    "f4_fp8q_2x3": dict(B=2, R=3, lengths=[3000, 4500], seed=507, fp8_query=True),
}


def _case(name):
    kw = dict(CASES[name])
    print(f"\n[case] mxfp4 {name} {kw}", flush=True)
    return make_case(name=name, key_format="mxfp4", **kw).to("cuda")


@pytest.mark.parametrize("name", sorted(CASES))
def test_mxfp4_scores_match_oracle(gpu, name):
    case = _case(name)
    scores = gpu_scores(case).cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        check_scores(scores[row, : pos[row] + 1], oracle.row_scores(case, row), f"{name} row {row}")
        assert np.all(np.isnan(scores[row, pos[row] + 1 :])), f"{name} row {row}: wrote past its position"


@pytest.mark.parametrize("name", ["f4_1x4_3k", "f4_2x3_perm"])
def test_mxfp4_topk_exact_and_in_band(gpu, name):
    case = _case(name)
    scores = gpu_scores(case, sentinel=0.0)
    idx = gpu_topk(scores, row_len_of(case), 2048).cpu().numpy()
    s = scores.cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        check_topk_exact(idx[row], s[row, : pos[row] + 1], 2048, f"{name} row {row}")
        check_topk_band(idx[row], oracle.row_scores(case, row), 2048, f"{name} row {row}")


@pytest.mark.parametrize("name", ["f4_1x4_3k", "f4_2x3_perm", "f4_1x8", "f4_fp8q_2x3"])
def test_mxfp4_fused_decode_matches_oracle(gpu, name):
    case = _case(name)
    out, lse, idx = gpu_decode(case)
    idx_h = idx.cpu().numpy()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    res = oracle.dsa_rows(case, idx=idx_h)
    for row in range(case.rows):
        check_topk_band(idx_h[row], res[row]["scores"], case.topk, f"{name} row {row}")
        check_attention(out[row], lse[row], res[row]["out"], res[row]["lse"], f"{name} row {row}")
