"""The no-allocation decode attention, dsa_sparse_mla_decode_noalloc (the
library's own static scratch for the split partials), against
dsa_sparse_mla_decode with a caller workspace, on the same selections.
Calls run back to back on shrinking inputs: 255 rows (the most scratch any
shape needs: two splits of 16 heads x 514 floats per row), then 16 rows
(eight splits), then 3 rows, so stale partials of a larger call must not
leak into a smaller one."""

import numpy as np
import pytest
import torch

import sparse_attention_index_amd as dsa
from tests.gpu_run import gpu_mla, gpu_scores, gpu_topk, row_len_of
from tests.parity import check_attention
from workloads import make_case

pytestmark = pytest.mark.gpu


def _noalloc(case, idx):
    rows = case.rows
    out = torch.full((rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_decode_noalloc(dsa.Batch.of(case), dsa.Cache.of(case), case.q_mla, idx, case.sm_scale,
                                      out, lse)
    return out, lse


def test_noalloc_decode_attention_matches_the_workspace_entry_point(gpu):
    cases = [
        make_case(85, 3, [2100 + 37 * b for b in range(85)], seed=301, permute_blocks=True, name="85x3"),
        make_case(4, 4, [9000, 3000, 6000, 700], seed=302, permute_blocks=True, name="4x4"),
        make_case(1, 3, [5000], seed=303, name="1x3"),
    ]
    assert dsa.dsa_workspace_size(dsa.DSA_WS_MLA_DECODE, 255, 0, 2048) == 16 << 20
    for case in cases:
        case = case.to("cuda")
        print(f"\n[no-alloc] {case.name} rows={case.rows}", flush=True)
        idx = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), case.topk)
        ref_out, ref_lse = gpu_mla(case, idx)
        out, lse = _noalloc(case, idx)
        torch.cuda.synchronize()
        ro, rl = ref_out.float().cpu().numpy(), ref_lse.cpu().numpy()
        go, gl = out.float().cpu().numpy(), lse.cpu().numpy()
        for row in range(case.rows):
            check_attention(go[row], gl[row], ro[row], rl[row], f"{case.name} row {row}")
        # the same kernels over the same selection: identical results
        assert np.array_equal(go, ro) and np.array_equal(gl, rl), case.name
