"""GPU parity of each stage and of the fused decode against the oracle.

Sizes are small enough for the float64 oracle to finish in seconds while
spanning several tiles, pages and workgroups, ragged lengths, permuted page
tables, partial last pages, 1-8 rows per request and both query precisions.
"""

import numpy as np
import pytest
import torch

import sparse_attention_index_amd as dsa

import oracle
from tests.gpu_run import gpu_decode, gpu_mla, gpu_scores, gpu_topk, row_len_of
from tests.parity import check_attention, check_scores, check_topk_band, check_topk_exact
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = {
    "1x1_8k": dict(B=1, R=1, lengths=[8192], seed=101),
    "2x4_ragged_perm": dict(B=2, R=4, lengths=[3000, 5001], seed=102, permute_blocks=True),
    "3x3_short_perm": dict(B=3, R=3, lengths=[700, 64, 4099], seed=103, permute_blocks=True),
    "1x8": dict(B=1, R=8, lengths=[2500], seed=104),
    "2x5": dict(B=2, R=5, lengths=[1000, 1300], seed=105),
    "2x7_perm": dict(B=2, R=7, lengths=[2900, 4100], seed=111, permute_blocks=True),
    "1x12": dict(B=1, R=12, lengths=[3100], seed=112),
    "1x2_tiny": dict(B=1, R=2, lengths=[130], seed=106),
    "fp8q_1x64": dict(B=1, R=64, lengths=[2048 + 64], seed=107, fp8_query=True),
    "fp8q_2x7": dict(B=2, R=7, lengths=[5000, 3333], seed=108, fp8_query=True, permute_blocks=True),
    # E4M3 query rows with one row per scoring wave (decode-sized requests)
    "fp8q_2x3_perm": dict(B=2, R=3, lengths=[4100, 1500], seed=125, fp8_query=True, permute_blocks=True),
}

# fused decode only: rows past the single-workgroup top-k path (sliced
# selection), with a row shorter than k, over permuted pages
FUSED_ONLY = {
    "2x2_long_perm": dict(B=2, R=2, lengths=[50000, 1500], seed=109, permute_blocks=True),
    # filtered decode (contexts past 40,960): ragged requests, one shorter than k,
    # scoring workgroups split in proportion to the lengths
    "5x3_filtered_ragged": dict(B=5, R=3, lengths=[41000, 60000, 1900, 45000, 90000], seed=113,
                                permute_blocks=True),
    # 160 rows: the smaller candidate buffer per row, few scoring workgroups
    # per request (a -inf threshold overflows their regions)
    "40x4_many_rows": dict(B=40, R=4, lengths=[45000 + 97 * b for b in range(40)], seed=114, device="cuda"),
    # filtered decode with seven verification rows per request (two rows per wave)
    "2x7_filtered": dict(B=2, R=7, lengths=[45000, 70001], seed=115, permute_blocks=True),
    # ten rows per request: the sampling pass's waves take a second row each
    "1x10_filtered": dict(B=1, R=10, lengths=[52000], seed=116, permute_blocks=True),
    # E4M3 index queries with row scales through the filtered decode: one row
    # per wave (with a request shorter than k), two rows per wave, two row
    # groups, and MXFP4 keys
    "fp8q_3x4_filtered": dict(B=3, R=4, lengths=[45000, 70000, 1900], seed=117, permute_blocks=True,
                              fp8_query=True),
    "fp8q_2x6_filtered": dict(B=2, R=6, lengths=[50000, 43000], seed=118, fp8_query=True),
    "fp8q_1x10_filtered": dict(B=1, R=10, lengths=[52000], seed=119, permute_blocks=True, fp8_query=True),
    "fp8q_mx_2x4_filtered": dict(B=2, R=4, lengths=[50000, 41500], seed=120, fp8_query=True, key_format="mxfp4"),
    # many E4M3 rows of one request (a prefill chunk's shape): 16 rows per
    # scoring workgroup, the sampling pass's row groups in its grid, and (at
    # 1,024 rows) so few scoring workgroups per row group that the selection
    # gathers each region with a group of waves
    "fp8q_1x64_filtered": dict(B=1, R=64, lengths=[50000], seed=121, permute_blocks=True, fp8_query=True),
    "fp8q_1x1024_filtered": dict(B=1, R=1024, lengths=[46000], seed=122, fp8_query=True),
    # MXFP4 keys past 8 rows per request: the sampling pass stages its pages in
    # LDS for each group of 8 rows; two rows per scoring wave (bf16 queries)
    # and 16 rows per scoring workgroup with 64 sampled pages (E4M3 queries)
    "mx_1x12_filtered": dict(B=1, R=12, lengths=[52000], seed=123, permute_blocks=True, key_format="mxfp4"),
    "fp8q_mx_1x40_filtered": dict(B=1, R=40, lengths=[47000], seed=124, fp8_query=True, key_format="mxfp4"),
    # E4M3 queries over MXFP4 keys with two rows per scoring wave
    "fp8q_mx_1x12_filtered": dict(B=1, R=12, lengths=[50000], seed=126, fp8_query=True, key_format="mxfp4"),
}


def _case(name, **over):
    kw = dict({**CASES, **FUSED_ONLY}[name])
    kw.update(over)
    print(f"\n[case] {name} {kw}", flush=True)
    return make_case(name=name, **kw).to("cuda")


@pytest.mark.parametrize("name", sorted(CASES))
def test_scores_match_oracle_and_respect_causality(gpu, name):
    case = _case(name)
    scores = gpu_scores(case).cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        ref = oracle.row_scores(case, row)
        check_scores(scores[row, : pos[row] + 1], ref, f"{name} row {row}")
        assert np.all(np.isnan(scores[row, pos[row] + 1 :])), f"{name} row {row}: wrote past its position"


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("k", [2048, 100])
def test_topk_exact_on_gpu_scores(gpu, name, k):
    case = _case(name)
    scores = gpu_scores(case, sentinel=0.0)
    idx = gpu_topk(scores, row_len_of(case), k).cpu().numpy()
    s = scores.cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        check_topk_exact(idx[row], s[row, : pos[row] + 1], k, f"{name} row {row}")


@pytest.mark.parametrize("name", ["1x1_8k", "2x4_ragged_perm", "fp8q_2x7"])
def test_topk_within_band_of_oracle_scores(gpu, name):
    case = _case(name)
    scores = gpu_scores(case, sentinel=0.0)
    idx = gpu_topk(scores, row_len_of(case), case.topk).cpu().numpy()
    for row in range(case.rows):
        check_topk_band(idx[row], oracle.row_scores(case, row), case.topk, f"{name} row {row}")


# Rows of at most this many scores are selected by the one-kernel path (whole
# row in registers); longer rows by the filter + final kernels.
SHORT_MAX = 40960


def _rows_tensor(rows, min_ld=0):
    L = max(max(len(r) for r in rows), min_ld, 1)
    ld = (L + 63) // 64 * 64
    t = torch.zeros((len(rows), ld), dtype=torch.float32)
    for i, r in enumerate(rows):
        t[i, : len(r)] = torch.as_tensor(r, dtype=torch.float32)
    return t.cuda(), torch.tensor([len(r) for r in rows], dtype=torch.int32).cuda()


@pytest.mark.parametrize("path", ["short", "long"])
def test_topk_edge_cases(gpu, path):
    rng = np.random.default_rng(7)
    rows = [
        np.zeros(10000),  # one bin, more ties than the candidate buffer: full-row path
        np.zeros(3000),  # one bin, ties resolved among candidates
        rng.standard_normal(1500),  # fewer than k: all + padding
        np.zeros(0),  # empty row: all padding
        rng.integers(0, 20, 20000).astype(np.float64),  # heavy ties at the threshold
        np.concatenate([-np.abs(rng.standard_normal(5000)), np.array([-0.0, 0.0] * 50)]),  # signs and zeros
        rng.standard_normal(70000) * 1e-30,  # tiny magnitudes
        np.full(4096, 3.25),  # exactly 2k ties
        np.where(rng.random(300000) < 0.01, 5.0 + rng.random(300000), rng.random(300000)),  # planted cluster
    ]
    if path == "short":
        rows = [r[:SHORT_MAX] for r in rows] + [rng.standard_normal(SHORT_MAX - 3)]  # partial last vector
    print(f"\n[case] topk edge rows ({path})", [len(r) for r in rows], flush=True)
    scores, row_len = _rows_tensor(rows, min_ld=0 if path == "short" else 2 * SHORT_MAX)
    assert (scores.shape[1] <= SHORT_MAX) == (path == "short")
    for k in (2048, 1, 1000):
        idx = gpu_topk(scores, row_len, k).cpu().numpy()
        s32 = scores.cpu().numpy()
        for i, r in enumerate(rows):
            check_topk_exact(idx[i], s32[i, : len(r)], k, f"edge row {i} k {k}")


@pytest.mark.parametrize("L", [SHORT_MAX - 3, 3 * SHORT_MAX + 5])
def test_topk_unaligned_rows(gpu, L):
    """Rows that start off a 16-byte boundary, with an odd row stride (the scalar-load variants)."""
    rng = np.random.default_rng(L)
    rows = 3
    base = torch.as_tensor(rng.standard_normal((rows, L + 2)), dtype=torch.float32).cuda()
    scores = base[:, 1 : L + 1]  # stride L + 2, first element 4 bytes past the allocation start
    lens = [L, L - 1, 3000]
    row_len = torch.tensor(lens, dtype=torch.int32).cuda()
    print(f"\n[case] topk unaligned L={L} stride={scores.stride(0)}", flush=True)
    for k in (2048, 7):
        ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, rows, scores.stride(0), k))
        idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(scores, row_len, k, idx, ws)
        idx_h, s = idx.cpu().numpy(), scores.cpu().numpy()
        for i, n in enumerate(lens):
            check_topk_exact(idx_h[i], s[i, :n], k, f"unaligned L {L} row {i} k {k}")


def test_topk_vector_path_reads_a_partial_last_vector(gpu):
    """16-byte-aligned rows with a row stride that is a multiple of 4 take the
    vector-load slice path; rows of 3 * 40,960 + 1, + 2 and + 3 scores end
    inside a 16-byte vector, and their largest scores sit in exactly those
    last 1-3 positions (the most recent tokens of a decode row). Checked
    through dsa_topk and through the DCP shard selection (shard rows end
    off a multiple of 4 too)."""
    rng = np.random.default_rng(41)
    rows = []
    for extra in (1, 2, 3):
        r = rng.standard_normal(3 * SHORT_MAX + extra)
        r[-extra:] = 100.0 + np.arange(extra)
        rows.append(r)
    rows.append(rng.standard_normal(3 * SHORT_MAX + 2))
    rows[-1][-1] = 50.0
    scores, row_len = _rows_tensor(rows)
    assert scores.data_ptr() % 16 == 0 and scores.stride(0) % 4 == 0
    print("\n[case] topk partial last vector", [len(r) for r in rows], flush=True)
    s32 = scores.cpu().numpy()
    for k in (2048, 3):
        idx = gpu_topk(scores, row_len, k).cpu().numpy()
        for i, r in enumerate(rows):
            check_topk_exact(idx[i], s32[i, : len(r)], k, f"tail row {i} k {k}")
            assert len(r) - 1 in set(idx[i].tolist()), f"tail row {i} k {k}: last position dropped"
    W, k = 2, 2048
    C = int(1.5 * k / W)
    nrows = len(rows)
    ws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_TOPK, nrows, scores.stride(0), k, W, C))
    idx = torch.full((nrows, k), -7, dtype=torch.int32, device="cuda")
    resend = torch.zeros((nrows, W), dtype=torch.uint8, device="cuda")
    dsa.dsa_dcp_topk(scores, row_len, k, W, C, idx, resend, ws)
    idx_h = idx.cpu().numpy()
    for i, r in enumerate(rows):
        check_topk_exact(idx_h[i], s32[i, : len(r)], k, f"dcp tail row {i}")


@pytest.mark.parametrize("aligned", [True, False])
def test_topk_survivors_clustered_in_few_slices(gpu, aligned):
    """Long rows whose high scores crowd into a few slices of the row: the
    survivors of those slices pass the slice workgroups' own candidate
    regions, and the final pass reads those slices again from the row. The
    clusters: the most recent 32,768 positions (the decode case), the first
    20,000, one across the middle, one of exact ties, and one dense enough to
    hold the whole top k. `aligned` False gives rows with an odd stride that
    start 4 bytes into the allocation (scalar loads)."""
    rng = np.random.default_rng(53)
    L = 1 << 20
    rows = []

    def planted(lo, hi, frac, value=None):
        r = rng.standard_normal(L)
        hit = lo + np.flatnonzero(rng.random(hi - lo) < frac)
        r[hit] = value if value is not None else 5.0 + rng.random(hit.size)
        return r

    rows.append(planted(L - 32768, L, 0.1))
    rows.append(planted(0, 20000, 0.1))
    rows.append(planted(L // 2 - 9000, L // 2 + 9000, 0.15))
    rows.append(planted(L - 32768, L, 0.1, value=7.0))
    rows.append(planted(L - 8192, L, 0.5))
    lens = [L, L, L - 1, L - 3, L]
    nrows = len(rows)
    if aligned:
        scores = torch.as_tensor(np.stack(rows), dtype=torch.float32).cuda()
        assert scores.data_ptr() % 16 == 0 and scores.stride(0) % 4 == 0
    else:
        base = torch.zeros((nrows, L + 3), dtype=torch.float32)
        base[:, 1 : L + 1] = torch.as_tensor(np.stack(rows), dtype=torch.float32)
        scores = base.cuda()[:, 1 : L + 1]
        assert scores.stride(0) % 2 == 1
    row_len = torch.tensor(lens, dtype=torch.int32).cuda()
    print(f"\n[case] topk clustered survivors aligned={aligned}", lens, flush=True)
    s32 = scores.cpu().numpy()
    for k in (2048, 500):
        ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, nrows, scores.stride(0), k))
        idx = torch.full((nrows, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(scores, row_len, k, idx, ws)
        idx_h = idx.cpu().numpy()
        for i, n in enumerate(lens):
            check_topk_exact(idx_h[i], s32[i, :n], k, f"clustered row {i} k {k}")


@pytest.mark.parametrize("min_ld", [0, 2 * SHORT_MAX])
def test_topk_all_ties_pick_lowest_positions(gpu, min_ld):
    scores, row_len = _rows_tensor([np.ones(9000), np.ones(2500)], min_ld=min_ld)
    idx = gpu_topk(scores, row_len, 2048).cpu().numpy()
    assert sorted(idx[0].tolist()) == list(range(2048))
    assert sorted(idx[1].tolist()) == list(range(2048))


@pytest.mark.parametrize("name", ["1x1_8k", "2x4_ragged_perm", "3x3_short_perm", "2x5", "fp8q_1x64"])
@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("k", [2048, 100])
def test_sparse_mla_matches_oracle_on_gpu_selection(gpu, name, split, k):
    case = _case(name)
    scores = gpu_scores(case, sentinel=0.0)
    idx = gpu_topk(scores, row_len_of(case), k)
    out, lse = gpu_mla(case, idx, split=split)
    out, lse, idx_h = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    for row in range(case.rows):
        ro, rl = oracle.dense_attend_row(case, row, idx_h[row])
        check_attention(out[row], lse[row], ro, rl, f"{name} row {row} split {split} k {k}")


def test_sparse_mla_short_context_equals_dense(gpu):
    case = _case("1x2_tiny")
    case2 = make_case(2, 4, [2048, 1000], seed=110, permute_blocks=True).to("cuda")
    for c in (case, case2):
        idx = gpu_topk(gpu_scores(c, sentinel=0.0), row_len_of(c), 2048)
        out, lse = gpu_mla(c, idx)
        pos = c.positions().numpy()
        for row in range(c.rows):
            ro, rl = oracle.dense_attend_row(c, row, np.arange(pos[row] + 1))
            check_attention(out[row].float().cpu().numpy(), lse[row].cpu().numpy(), ro, rl, f"dense row {row}")


def test_sparse_mla_skips_invalid_entries(gpu):
    case = _case("2x4_ragged_perm")
    rng = np.random.default_rng(3)
    pos = case.positions().numpy()
    k = 300
    idx = np.full((case.rows, k), -1, np.int32)
    for row in range(case.rows):
        if row == 3:
            continue  # an all-invalid row
        sel = rng.choice(pos[row] + 1, size=200, replace=False)
        slots = rng.choice(k, size=200, replace=False)
        idx[row, slots] = sel
    idx_t = torch.from_numpy(idx).cuda()
    for split in (True, False):
        out, lse = gpu_mla(case, idx_t, split=split)
        out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
        for row in range(case.rows):
            ro, rl = oracle.dense_attend_row(case, row, idx[row])
            check_attention(out[row], lse[row], ro, rl, f"holes row {row} split {split}")
        assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))


@pytest.mark.parametrize("name", ["1x1_8k", "2x4_ragged_perm", "3x3_short_perm", "1x8", "2x2_long_perm",
                                  "fp8q_2x3_perm", "5x3_filtered_ragged", "2x7_filtered", "1x10_filtered", "fp8q_2x7",
                                  "fp8q_3x4_filtered", "fp8q_2x6_filtered", "fp8q_1x10_filtered",
                                  "fp8q_mx_2x4_filtered", "fp8q_1x64_filtered", "mx_1x12_filtered",
                                  "fp8q_mx_1x40_filtered", "fp8q_mx_1x12_filtered"])
def test_fused_decode_matches_oracle_and_stages(gpu, name):
    case = _case(name)
    out, lse, idx = gpu_decode(case)
    # stage-by-stage run of the same kernels selects the identical set
    s_idx = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), case.topk).cpu().numpy()
    idx_h = idx.cpu().numpy()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    res = oracle.dsa_rows(case, idx=idx_h)
    for row in range(case.rows):
        assert set(idx_h[row].tolist()) == set(s_idx[row].tolist()), f"{name} row {row}: fused vs staged"
        check_topk_band(idx_h[row], res[row]["scores"], case.topk, f"{name} row {row}")
        check_attention(out[row], lse[row], res[row]["out"], res[row]["lse"], f"{name} row {row}")


def _wide_range(t, seed, span=24):
    """Each bf16 element scaled by 2^-e, e uniform in 0..span: every query head
    then spans far more than 2^10 in magnitude (the split of a bf16 query
    into two E4M3 terms under one power-of-two scale per head is exact only
    down to ~2^-10 of the head's largest element)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    e = torch.randint(0, span + 1, tuple(t.shape), generator=g).float()
    return (t.float().cpu() * torch.exp2(-e)).to(torch.bfloat16).to(t.device)


def _head_range(t):
    a = t.float().abs().cpu()
    a = a.reshape(-1, a.shape[-1])
    nz = torch.where(a > 0, a, torch.full_like(a, float("inf")))
    return (a.max(dim=1).values / nz.min(dim=1).values).min().item()


def test_query_heads_with_wide_dynamic_range(gpu):
    case = _case("2x4_ragged_perm")
    case.q_idx = _wide_range(case.q_idx, 1)
    case.q_mla = _wide_range(case.q_mla, 2)
    assert _head_range(case.q_idx) > 2.0**16 and _head_range(case.q_mla) > 2.0**16
    scores = gpu_scores(case).cpu().numpy()
    pos = case.positions().numpy()
    for row in range(case.rows):
        check_scores(scores[row, : pos[row] + 1], oracle.row_scores(case, row), f"wide-range scores row {row}")
    idx = gpu_topk(torch.from_numpy(np.nan_to_num(scores, nan=0.0)).cuda(), row_len_of(case), case.topk)
    out, lse = gpu_mla(case, idx)
    out, lse, idx_h = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    for row in range(case.rows):
        ro, rl = oracle.dense_attend_row(case, row, idx_h[row])
        check_attention(out[row], lse[row], ro, rl, f"wide-range attention row {row}")
    f_out, f_lse, f_idx = gpu_decode(case)
    f_idx = f_idx.cpu().numpy()
    res = oracle.dsa_rows(case, idx=f_idx)
    f_out, f_lse = f_out.float().cpu().numpy(), f_lse.cpu().numpy()
    for row in range(case.rows):
        check_topk_band(f_idx[row], res[row]["scores"], case.topk, f"wide-range fused row {row}")
        check_attention(f_out[row], f_lse[row], res[row]["out"], res[row]["lse"], f"wide-range fused row {row}")


def _kth_scores(case, k):
    """Each row's k-th largest fp32 score on the GPU (-inf for rows of fewer than k)."""
    s = gpu_scores(case, sentinel=float("-inf"))
    n = s.shape[1]
    return torch.topk(s, min(k, n), dim=1).values[:, -1].contiguous()


@pytest.mark.parametrize("name", ["2x2_long_perm", "5x3_filtered_ragged", "1x1_8k", "40x4_many_rows", "2x7_filtered",
                                  "1x10_filtered", "fp8q_3x4_filtered", "fp8q_2x6_filtered", "fp8q_1x64_filtered",
                                  "mx_1x12_filtered"])
def test_thresholded_decode_equals_the_staged_path_whatever_the_threshold(gpu, name):
    """The filtered decode with caller-given thresholds against the stored
    path (dsa_index_score -> dsa_topk -> dsa_sparse_mla_decode). Too high a
    threshold (+inf, NaN, just above the k-th score: fewer than k
    candidates) sends rows to the exact fallback (full scores, whole-row
    selection); -inf keeps every score (selected from a compacted copy past
    what LDS holds, or, where a workgroup's region overflows, by the
    fallback); exactly the k-th score decides from the candidates. Every
    variant, and a per-row mix of them, selects the staged set."""
    case = _case(name)
    k = case.topk
    ref_idx = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), k)
    ref_out, ref_lse = gpu_mla(case, ref_idx)
    ref_idx = ref_idx.cpu().numpy()
    kth = _kth_scores(case, k)
    rows = case.rows
    above = torch.nextafter(kth, torch.full_like(kth, float("inf")))
    mix = torch.where(torch.arange(rows, device="cuda") % 3 == 0, above,
                      torch.where(torch.arange(rows, device="cuda") % 3 == 1, kth, torch.full_like(kth, -1e30)))
    variants = {
        "+inf": torch.full((rows,), float("inf"), device="cuda"),
        "-inf": torch.full((rows,), float("-inf"), device="cuda"),
        "nan": torch.full((rows,), float("nan"), device="cuda"),
        "kth": kth,
        "above_kth": above,
        "mixed": mix,
    }
    ro, rl = ref_out.float().cpu().numpy(), ref_lse.cpu().numpy()
    for label, thr in variants.items():
        print(f"[thresholded] {name} {label}", flush=True)
        out, lse, idx = gpu_decode(case, threshold=thr)
        idx = idx.cpu().numpy()
        for row in range(rows):
            assert set(idx[row].tolist()) == set(ref_idx[row].tolist()), f"{name} {label} row {row}"
        check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"{name} {label}")


@pytest.mark.parametrize("name", ["2x2_long_perm", "5x3_filtered_ragged", "2x4_ragged_perm", "40x4_many_rows",
                                  "2x7_filtered", "1x10_filtered", "fp8q_3x4_filtered", "fp8q_1x10_filtered",
                                  "fp8q_mx_2x4_filtered", "fp8q_1x64_filtered", "fp8q_1x1024_filtered",
                                  "mx_1x12_filtered", "fp8q_mx_1x40_filtered", "fp8q_mx_1x12_filtered"])
def test_filter_stage_entry_points_select_the_stored_top_k(gpu, name):
    """dsa_filter_threshold -> dsa_filter_score -> dsa_filter_select, called
    one by one on a workspace that starts with stale bytes, select exactly
    dsa_topk's set over dsa_index_score's scores: with sampled thresholds,
    with each row's k-th score as the caller's threshold, and with +inf (every
    row through the fallback). 2x4_ragged_perm is short enough that the fused
    decode would not filter it; the stages filter whatever the length."""
    case = _case(name)
    k = case.topk
    ref = gpu_topk(gpu_scores(case, sentinel=0.0), row_len_of(case), k).cpu().numpy()
    b, c = dsa.Batch.of(case), dsa.Cache.of(case)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, case.rows, case.max_ctx, k))
    kth = _kth_scores(case, k)
    for label, thr in (("sampled", None), ("kth", kth), ("+inf", torch.full_like(kth, float("inf")))):
        print(f"[filter stages] {name} {label}", flush=True)
        ws.fill_(0xA5)
        idx = torch.full((case.rows, k), -7, dtype=torch.int32, device="cuda")
        qs = case.q_idx_scale
        dsa.dsa_filter_threshold(b, c, case.q_idx, case.w, k, ws, threshold=thr, q_scale=qs)
        dsa.dsa_filter_score(b, c, case.q_idx, case.w, k, ws, q_scale=qs)
        dsa.dsa_filter_select(b, c, case.q_idx, case.w, k, idx, ws, q_scale=qs)
        got = idx.cpu().numpy()
        for row in range(case.rows):
            assert set(got[row].tolist()) == set(ref[row].tolist()), f"{name} {label} row {row}"


def test_filter_stages_refuse_requests_past_the_selection_capacity(gpu):
    """One row at 140M tokens would spread its request over more than 1,024
    scoring workgroups (each stages at most 2,048 page ids, and the
    selection has one thread per workgroup): the filtered stages and the
    thresholded decode refuse it on the host, before any kernel runs (the
    cache holds one zero page that every table entry points to)."""
    L = 140 << 20
    dev = "cuda"
    b = dsa.Batch(1, torch.tensor([L], dtype=torch.int32, device=dev),
                  torch.zeros((1, (L + 63) // 64), dtype=torch.int32, device=dev), L)
    c = dsa.Cache(torch.zeros((1, 64, 128), dtype=torch.uint8, device=dev), torch.ones(64, device=dev),
                  torch.zeros((1, 64, 576), dtype=torch.uint8, device=dev), torch.ones(64, device=dev))
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((1, 32), dtype=torch.bfloat16, device=dev)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, 1, L, 2048))
    for call in (lambda: dsa.dsa_filter_threshold(b, c, q, w, 2048, ws),
                 lambda: dsa.dsa_filter_score(b, c, q, w, 2048, ws),
                 lambda: dsa.dsa_filter_select(b, c, q, w, 2048, torch.empty((1, 2048), dtype=torch.int32,
                                                                             device=dev), ws)):
        with pytest.raises(dsa.DsaError) as err:
            call()
        assert err.value.status == dsa.DSA_ERR_UNSUPPORTED and "1024 scoring workgroups" in str(err.value)
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device=dev)
    with pytest.raises(dsa.DsaError) as err:
        dsa.dsa_decode(b, c, q, w, torch.zeros((1, 16, 576), dtype=torch.bfloat16, device=dev), 2048, 0.04, out,
                       ws=ws, threshold=torch.zeros(1, device=dev))
    assert err.value.status == dsa.DSA_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_fused_decode_selection_is_deterministic(gpu):
    case = _case("2x4_ragged_perm")
    a = gpu_decode(case)
    b = gpu_decode(case)
    ia, ib = a[2].cpu().numpy(), b[2].cpu().numpy()
    for row in range(case.rows):
        assert set(ia[row].tolist()) == set(ib[row].tolist())
    check_attention(a[0].float().cpu().numpy(), a[1].cpu().numpy(), b[0].float().cpu().numpy(),
                    b[1].cpu().numpy(), "repeat")


def test_binding_rejects_mismatched_tensors_before_launch(gpu):
    """Without row scales the fused decode takes bf16 indexer queries: E4M3
    query codes (half the bytes) passed without q_scale must be refused by
    the binding before any kernel reads them."""
    case = _case("fp8q_2x7")
    rows, k = case.rows, case.topk
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="q_idx"):
        dsa.dsa_decode(dsa.Batch.of(case), dsa.Cache.of(case), case.q_idx, case.w, case.q_mla, k, case.sm_scale,
                       out, None, None, ws)
    scores = torch.empty((rows, 64), dtype=torch.float32, device="cuda")  # narrower than the context
    with pytest.raises(ValueError, match="scores"):
        dsa.dsa_index_score(dsa.Batch.of(case), dsa.Cache.of(case), case.q_idx, case.w, scores,
                            q_scale=case.q_idx_scale)
