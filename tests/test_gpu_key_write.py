"""GPU parity of the index-key write (dsa_index_key_write) against the oracle.

The oracle normalises in float64 and takes the quantisation decision in
float32; the kernel normalises in float32. So:
* scales agree to float32 rounding of the normalisation (relative 4e-6);
* a code may differ from the oracle's only where the exact value lies within
  rounding of an E4M3 midpoint, and then it must be the other neighbour: the
  GPU's code is checked to be (up to 1e-5 relative) as near to the exact
  value as the oracle's;
* every slot that no new row targets is left byte-for-byte unchanged.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_index_amd as dsa
from tests.gpu_run import gpu_scores
from tests.parity import check_scores
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = {
    "1x1": dict(B=1, R=1, lengths=[700], seed=301),
    "3x4_perm": dict(B=3, R=4, lengths=[130, 64, 4099], seed=302, permute_blocks=True),
    "2x8": dict(B=2, R=8, lengths=[1000, 257], seed=303),
    "prefill_512": dict(B=1, R=512, lengths=[512 + 3000], seed=304),
}


def _keys(rows, seed, mean=0.3, std=2.0):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn((rows, 128), generator=g) * std + mean).to(torch.bfloat16)
    w = (1.0 + 0.25 * torch.randn(128, generator=g)).float()
    b = (0.1 * torch.randn(128, generator=g)).float()
    return k, w, b


def _run(case, k, w, b, eps):
    kf = case.key_fp8.clone()
    ks = case.key_scale.clone()
    dsa.dsa_index_key_write(dsa.Batch.of(case), k.cuda(), w.cuda(), b.cuda(), kf, ks, eps=eps)
    torch.cuda.synchronize()
    return kf.cpu().numpy(), ks.cpu().numpy()


def _expected(case, k, w, b, eps):
    host = case.to("cpu")
    slots = oracle.write_slots(host.ctx_len.numpy(), host.block_table.numpy(), case.R, host.key_fp8.shape[0])
    y = oracle.layer_norm(k.double().numpy(), w.double().numpy(), b.double().numpy(), eps)
    codes, scales = oracle.quantize_rows(y)
    planes = oracle.scatter_rows(host.key_fp8.numpy(), host.key_scale.numpy(), codes, scales, slots)
    return slots, y, codes, scales, planes


def _check(case, k, w, b, eps, name):
    gk, gs = _run(case, k, w, b, eps)
    slots, y, codes, scales, (ek, es) = _expected(case, k, w, b, eps)
    tab = oracle.e4m3_table()
    written = np.zeros(ek.shape[:2], bool)
    for row, slot in enumerate(slots.tolist()):
        if slot < 0:
            continue
        blk, off = slot // 64, slot % 64
        written[blk, off] = True
        assert abs(gs[blk, off] - scales[row]) <= 4e-6 * scales[row], f"{name} row {row}: scale"
        diff = np.nonzero(gk[blk, off] != codes[row])[0]
        if diff.size:
            exact = y[row, diff] / scales[row]
            d_gpu = np.abs(tab[gk[blk, off, diff]] - exact)
            d_ref = np.abs(tab[codes[row, diff]] - exact)
            assert np.all(d_gpu <= d_ref + 1e-5 * np.abs(exact) + 1e-30), f"{name} row {row}: codes {diff.tolist()}"
    assert np.array_equal(gk[~written], ek[~written]), f"{name}: an untargeted key slot changed"
    assert np.array_equal(gs[~written], es[~written]), f"{name}: an untargeted scale slot changed"
    return int(written.sum())


@pytest.mark.parametrize("name", sorted(CASES))
def test_key_write_matches_oracle(gpu, name):
    case = make_case(name=name, device="cuda", **CASES[name])
    k, w, b = _keys(case.rows, CASES[name]["seed"])
    print(f"\n[case] key write {name} rows={case.rows}", flush=True)
    n = _check(case, k, w, b, 1e-6, name)
    assert n == case.rows  # every row's position is valid here


def test_key_write_edge_rows(gpu):
    case = make_case(B=2, R=4, lengths=[300, 64], seed=305, device="cuda")
    case.ctx_len[1] = 2  # 4 new rows but only 2 tokens: positions -2 and -1 are skipped
    k, w, b = _keys(case.rows, 305)
    k[0] = 5.0  # constant row: y = bias
    k[1] = 0.0
    b0 = torch.zeros(128)
    print("\n[case] key write edge rows", flush=True)
    n = _check(case, k, w, b, 1e-6, "edge")
    assert n == case.rows - 2
    # constant rows with zero bias: an all-zero normalised row has scale 1 and zero codes
    gk, gs = _run(case, k, w, b0, 1e-6)
    host = case.to("cpu")
    slot = oracle.write_slots(host.ctx_len.numpy(), host.block_table.numpy(), case.R, host.key_fp8.shape[0])[0]
    assert gs[slot // 64, slot % 64] == 1.0 and not gk[slot // 64, slot % 64].any()


def test_key_write_skips_rows_without_a_page(gpu):
    case = make_case(B=1, R=2, lengths=[200], seed=306, device="cuda")
    case.block_table[0, 3] = -1  # positions 198, 199 live in block 3
    k, w, b = _keys(case.rows, 306)
    print("\n[case] key write without page", flush=True)
    assert _check(case, k, w, b, 1e-6, "nopage") == 0


def test_written_keys_score_like_the_oracle(gpu):
    """Round trip: keys written by the kernel are read back by the scorer."""
    case = make_case(B=2, R=4, lengths=[1500, 900], seed=307, device="cuda")
    k, w, b = _keys(case.rows, 307)
    print("\n[case] key write then score", flush=True)
    dsa.dsa_index_key_write(dsa.Batch.of(case), k.cuda(), w.cuda(), b.cuda(), case.key_fp8, case.key_scale)
    scores = gpu_scores(case).cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        check_scores(scores[row, : pos[row] + 1], oracle.row_scores(case, row), f"written keys row {row}")
