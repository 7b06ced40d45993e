"""GPU parity of the decode-context-parallel simulation: the merged top-k
across W virtual shards must be exactly the single-device selection (and the
oracle's merge, resend flags included), and the LSE combine of the shards'
partial attention must match single-device attention and the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_index_amd as dsa
from tests.gpu_run import gpu_mla, gpu_scores, gpu_topk, row_len_of
from tests.parity import check_attention, sel_set
from workloads import make_case

pytestmark = pytest.mark.gpu

LENS = [5, 700, 2047, 2049, 9000, 40000, 3]


def _rows(kind, seed):
    g = torch.Generator().manual_seed(seed)
    ld = 40960
    s = torch.randn((len(LENS), ld), generator=g)
    if kind == "ties":
        s = torch.randint(0, 4, (len(LENS), ld), generator=g).float()
    elif kind == "zeros":
        s = torch.zeros((len(LENS), ld))
    elif kind == "shard0":
        s[:, 0::8] += 10.0  # every winner on shard 0 of 8 (and on the shards 0 mod 8 maps to for smaller W)
    return s.cuda(), torch.tensor(LENS, dtype=torch.int32).cuda()


def _dcp(scores, row_len, k, W, C):
    rows, ld = scores.shape
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    resend = torch.full((rows, W), 9, dtype=torch.uint8, device="cuda")
    ws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_TOPK, rows, ld, k, W, C))
    dsa.dsa_dcp_topk(scores, row_len, k, W, C, idx, resend, ws)
    return idx, resend


@pytest.mark.parametrize("kind", ["random", "ties", "zeros", "shard0"])
@pytest.mark.parametrize("W", [2, 4, 8])
@pytest.mark.parametrize("k", [2048, 100])
def test_dcp_topk_is_the_single_device_selection(gpu, kind, W, k):
    print(f"\n[case] dcp topk {kind} W={W} k={k}", flush=True)
    scores, row_len = _rows(kind, 11 + W)
    C = max(1, int(1.5 * k / W))
    idx, resend = _dcp(scores, row_len, k, W, C)
    single = gpu_topk(scores, row_len, k).cpu().numpy()
    idx, resend = idx.cpu().numpy(), resend.cpu().numpy()
    s = scores.cpu().numpy()
    for r, n in enumerate(LENS):
        got = sel_set(idx[r], n)
        assert got == sel_set(single[r], n), f"{kind} W={W} k={k} row {r}: differs from the single device"
        assert np.all(idx[r][min(k, n):] == -1), f"row {r}: padding"
        sel, rs, _ = oracle.dcp_select(s[r, :n].astype(np.float64), W, k, C)
        assert got == set(sel.tolist()), f"row {r}: differs from the oracle's merge"
        assert resend[r].astype(bool).tolist() == rs.tolist(), f"row {r}: resend {resend[r]} vs {rs.astype(int)}"


def test_dcp_topk_resends_when_one_shard_holds_the_winners(gpu):
    scores, row_len = _rows("shard0", 3)
    idx, resend = _dcp(scores, row_len, 2048, 8, 384)
    resend = resend.cpu().numpy()
    long_rows = [r for r, n in enumerate(LENS) if n >= 9000]
    for r in long_rows:
        assert resend[r].tolist() == [1] + [0] * 7


@pytest.mark.parametrize("W", [2, 8])
def test_dcp_attention_matches_single_device_and_oracle(gpu, W):
    case = make_case(2, 3, [5000, 1500], seed=601, permute_blocks=True).to("cuda")
    print(f"\n[case] dcp mla W={W}", flush=True)
    idx = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), 2048)
    rows, k = idx.shape
    out = torch.full((rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device="cuda")
    ws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_MLA, rows, 0, k, W))
    dsa.dsa_dcp_mla_decode(dsa.Batch.of(case), dsa.Cache.of(case), case.q_mla, idx, W, case.sm_scale, out, lse, ws)
    s_out, s_lse = gpu_mla(case, idx)
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    check_attention(out, lse, s_out.float().cpu().numpy(), s_lse.cpu().numpy(), f"W={W} vs single device")
    ih = idx.cpu().numpy()
    for row in range(rows):
        parts = [oracle.dense_attend_row(case, row, np.where(ih[row] % W == w, ih[row], -1)) for w in range(W)]
        ro, rl = oracle.lse_combine([p[0] for p in parts], [p[1] for p in parts])
        check_attention(out[row], lse[row], ro, rl, f"W={W} row {row} vs oracle")


def test_dcp_attention_with_shards_that_own_nothing(gpu):
    case = make_case(1, 2, [40], seed=602).to("cuda")  # 40 tokens over 64 shards: most own nothing
    idx = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), 2048)
    rows, k = idx.shape
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, 16), dtype=torch.float32, device="cuda")
    ws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_MLA, rows, 0, k, 64))
    dsa.dsa_dcp_mla_decode(dsa.Batch.of(case), dsa.Cache.of(case), case.q_mla, idx, 64, case.sm_scale, out, lse, ws)
    ih = idx.cpu().numpy()
    for row in range(rows):
        ro, rl = oracle.dense_attend_row(case, row, ih[row])
        check_attention(out[row].float().cpu().numpy(), lse[row].cpu().numpy(), ro, rl, f"row {row}")
