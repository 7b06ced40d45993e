"""Pins of the oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: the OCP E4M3 definition and
torch's own float8_e4m3fn cast, algebraic identities of ReLU, hand-worked
examples, heapq and torch's scaled_dot_product_attention as independent
library routines, and the byte figures the pages print.
"""

import heapq
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import traffic
from workloads import make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- FP8 decode


def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(tab[~nan], ref[~nan])


def test_e4m3_spec_points():
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0  # largest finite magnitude
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0**-6  # smallest normal
    assert t[0x01] == 2.0**-9  # smallest subnormal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0


# ---------------------------------------------------------------- scoring


def _rand_inputs(rng, n=257, H=32, D=128):
    q = rng.standard_normal((H, D))
    w = rng.uniform(0, 1, H)
    codes = rng.integers(0, 256, (n, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00  # no NaN codes
    scale = rng.uniform(0.001, 0.02, n)
    return q, w, oracle.dequant(codes, scale)


def test_scores_relu_difference_identity():
    # relu(x) - relu(-x) = x, so s(q) - s(-q) is linear: (sum_h w_h q_h) . k
    rng = np.random.default_rng(1)
    q, w, k = _rand_inputs(rng)
    lhs = oracle.index_scores(q, w, k) - oracle.index_scores(-q, w, k)
    rhs = k @ (w @ q)
    assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-12)


def test_scores_relu_sum_identity():
    # relu(x) + relu(-x) = |x|
    rng = np.random.default_rng(2)
    q, w, k = _rand_inputs(rng)
    lhs = oracle.index_scores(q, w, k) + oracle.index_scores(-q, w, k)
    rhs = np.abs(k @ q.T) @ w
    assert np.allclose(lhs, rhs, rtol=1e-12)


def test_scores_hand_worked_example():
    # Three active heads, two keys; every other head has q = 0.
    #   head 0: q = 2 e0,  w = 0.25 ; head 1: q = -e0, w = 1 ; head 5: q = 0.5 e3, w = 4
    #   key 0 codes: 3.0 at d0, 1.0 at d3, scale 1   -> dots (6, -3, 0.5)
    #        score = 0.25*6 + 0 + 4*0.5 = 3.5
    #   key 1 codes: -2.0 at d0, 4.0 at d3, scale .5 -> khat (-1, 0, 0, 2), dots (-2, 1, 1)
    #        score = 0 + 1*1 + 4*1 = 5.0
    q = np.zeros((32, 128))
    q[0, 0] = 2.0
    q[1, 0] = -1.0
    q[5, 3] = 0.5
    w = np.ones(32)
    w[0], w[1], w[5] = 0.25, 1.0, 4.0
    codes = np.zeros((2, 128), np.uint8)
    codes[0, 0], codes[0, 3] = 0x44, 0x38  # 3.0, 1.0
    codes[1, 0], codes[1, 3] = 0xC0, 0x48  # -2.0, 4.0
    k = oracle.dequant(codes, np.array([1.0, 0.5]))
    assert np.array_equal(oracle.index_scores(q, w, k), np.array([3.5, 5.0]))


def test_scores_homogeneous_and_linear_in_weights():
    rng = np.random.default_rng(3)
    q, w, k = _rand_inputs(rng)
    w2 = rng.uniform(0, 1, 32)
    s = oracle.index_scores(q, w, k)
    assert np.allclose(oracle.index_scores(2.5 * q, w, k), 2.5 * s, rtol=1e-12)
    assert np.allclose(oracle.index_scores(q, w + w2, k),
                       s + oracle.index_scores(q, w2, k), rtol=1e-12)
    # a positive per-token scale factors out of the ReLU
    assert np.allclose(oracle.index_scores(q, w, 3.0 * k), 3.0 * s, rtol=1e-12)
    # ... token by token, and a positive query-row scale likewise: applying
    # both scales after the ReLU (as a kernel may) equals the definition,
    # which applies them inside it
    c = rng.uniform(0.01, 5.0, k.shape[0])
    assert np.allclose(oracle.index_scores(0.7 * q, w, c[:, None] * k), 0.7 * c * s, rtol=1e-12)
    # a negative scale does not factor out: the scales must be positive
    assert not np.allclose(oracle.index_scores(q, w, -k), -s)


def test_scores_opposed_key_is_zero():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(128)
    q = np.tile(v, (32, 1))
    assert np.all(oracle.index_scores(q, np.ones(32), -v[None, :]) == 0.0)


# ---------------------------------------------------------------- selection


def _heap_topk(s, k):
    return set(heapq.nlargest(k, range(len(s)), key=lambda j: (s[j], -j)))


@pytest.mark.parametrize("n,k", [(5000, 2048), (2048, 2048), (700, 2048), (1, 2048), (3000, 64)])
def test_topk_matches_heapq_with_ties(n, k):
    rng = np.random.default_rng(n + k)
    s = rng.integers(0, 20, n).astype(np.float64)  # many ties
    got = oracle.topk_positions(s, k)
    assert len(got) == min(k, n) and len(set(got.tolist())) == len(got)
    assert set(got.tolist()) == _heap_topk(s, k)


def test_topk_planted_winners():
    rng = np.random.default_rng(5)
    s = rng.uniform(0, 1, 100000)
    win = rng.choice(100000, 2048, replace=False)
    s[win] = 2.0 + rng.uniform(0, 1, 2048)
    got = oracle.topk_positions(s, 2048)
    assert set(got.tolist()) == set(win.tolist())
    assert np.all(np.diff(s[got]) <= 0)  # rank order


def test_topk_separates_selected_from_rest():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(40000)
    got = oracle.topk_positions(s, 2048)
    rest = np.setdiff1d(np.arange(s.size), got)
    assert s[got].min() >= s[rest].max()


# ---------------------------------------------------------------- attention


def _rand_latents(rng, n):
    codes = rng.integers(0, 256, (n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    return oracle.dequant(codes, rng.uniform(0.001, 0.01, n))


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((16, 576))
    rows = _rand_latents(rng, 300)
    sm = 1.0 / math.sqrt(576)
    out, lse = oracle.attend(q, rows, sm)
    tq = torch.from_numpy(q)[:, None, :]  # [16, 1, 576]
    tk = torch.from_numpy(rows)[None].expand(16, -1, -1)
    tv = torch.from_numpy(rows[:, :512])[None].expand(16, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sm)[:, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    ref_lse = torch.logsumexp(sm * (torch.from_numpy(q) @ torch.from_numpy(rows).T), dim=1).numpy()
    assert np.allclose(lse, ref_lse, rtol=1e-12)


def test_attend_single_row_and_zero_query():
    rng = np.random.default_rng(8)
    rows = _rand_latents(rng, 37)
    q = rng.standard_normal((16, 576))
    out, lse = oracle.attend(q, rows[:1], 0.1)
    assert np.allclose(out, np.tile(rows[0, :512], (16, 1)), rtol=1e-13)
    assert np.allclose(lse, 0.1 * q @ rows[0], rtol=1e-12)
    out, lse = oracle.attend(np.zeros((16, 576)), rows, 0.1)
    assert np.allclose(out, np.tile(rows[:, :512].mean(axis=0), (16, 1)), rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, math.log(37), rtol=1e-13)


def test_attend_order_invariant_and_empty():
    rng = np.random.default_rng(9)
    rows = _rand_latents(rng, 64)
    q = rng.standard_normal((16, 576))
    perm = rng.permutation(64)
    a = oracle.attend(q, rows, 0.05)
    b = oracle.attend(q, rows[perm], 0.05)
    assert np.allclose(a[0], b[0], rtol=1e-12) and np.allclose(a[1], b[1], rtol=1e-13)
    out, lse = oracle.attend(q, rows[:0], 0.05)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- whole path


def test_short_context_sparse_equals_dense():
    case = make_case(2, 3, [1500, 2048], seed=11)
    res = oracle.dsa_rows(case)
    pos = case.positions().numpy()
    for row, r in res.items():
        assert sorted(r["sel"].tolist()) == list(range(pos[row] + 1))
        dense_out, dense_lse = oracle.dense_attend_row(case, row, np.arange(pos[row] + 1))
        assert np.allclose(r["out"], dense_out, rtol=1e-12, atol=1e-14)
        assert np.allclose(r["lse"], dense_lse, rtol=1e-13)


def test_causal_rows_never_see_later_tokens():
    # Plant an overwhelming key at the position of row 1; row 0 must not see it,
    # rows 1..3 must rank it first.
    case = make_case(1, 4, [5000], seed=12, topk=64)
    pos = case.positions().numpy()
    p = int(pos[1])
    blk, slot = int(case.block_table[0, p // 64]), p % 64
    direction = (case.w[1].float()[:, None] * case.q_idx[1].float()).sum(0)
    codes = torch.where(direction > 0, torch.tensor(0x7E), torch.tensor(0xFE)).to(torch.uint8)
    case.key_fp8[blk, slot] = codes
    case.key_scale[blk, slot] = 10.0
    res = oracle.dsa_rows(case)
    assert res[0]["scores"].size == pos[0] + 1
    assert p not in res[0]["sel"].tolist()
    for row in (1, 2, 3):
        assert res[row]["scores"].size == pos[row] + 1
        assert res[row]["sel"][0] == p


def test_paged_layout_does_not_change_results():
    a = make_case(3, 2, [700, 1300, 2600], seed=13, topk=256)
    b = make_case(3, 2, [700, 1300, 2600], seed=13, topk=256, permute_blocks=True)
    # same draws, different physical placement
    for name in ("q_idx", "w", "q_mla"):
        assert torch.equal(getattr(a, name), getattr(b, name))
    assert not torch.equal(a.block_table, b.block_table)
    ra, rb = oracle.dsa_rows(a), oracle.dsa_rows(b)
    for row in ra:
        assert np.array_equal(ra[row]["scores"], rb[row]["scores"])
        assert np.array_equal(ra[row]["sel"], rb[row]["sel"])
        assert np.array_equal(ra[row]["out"], rb[row]["out"])


def test_fp8_query_rows_dequantise_with_their_scale():
    case = make_case(1, 8, [600], seed=14, fp8_query=True, topk=128)
    s = oracle.row_scores(case, 3)
    q = oracle.e4m3_decode(case.q_idx[3].numpy()) * float(case.q_idx_scale[3])
    pos = int(case.positions()[3])
    k = oracle.dequant(case.key_fp8.reshape(-1, 128)[: pos + 1].numpy(),
                       case.key_scale.reshape(-1)[: pos + 1].numpy())
    # identity block table, so the first pos+1 pool rows are the request's tokens
    lin = k @ (case.w[3].float().numpy().astype(np.float64) @ q)
    s_neg = oracle.index_scores(-q, case.w[3].float().numpy(), k)
    assert np.allclose(s - s_neg, lin, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- bytes


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v, tol = line.split()
                vals[k] = (float(v), float(tol))
    return vals


def _close(x, ref):
    v, tol = ref
    return abs(x - v) <= tol * abs(v)


def test_byte_model_reproduces_the_pages_figures():
    g = _golden("page_byte_figures.txt")
    n = 128 * 1024
    dense = traffic.dense_mla_bytes(n)
    dsa_noscores = traffic.dsa_bytes(n, score_bytes=0)
    scores = n * traffic.SCORE_BYTES
    assert _close(dense, g["dense_128k_bytes"])
    assert _close(dsa_noscores, g["dsa_128k_bytes_no_scores"])
    assert _close(scores, g["scores_128k_bytes"])
    assert _close(dense / traffic.dsa_bytes(n), g["ratio_128k_1row"])
    assert _close(dense / traffic.dsa_bytes(n, rows=4), g["ratio_128k_4rows"])
    r1m = traffic.dense_mla_bytes(1 << 20) / traffic.dsa_bytes(1 << 20)
    assert g["ratio_1m_1row_min"][0] < r1m < g["ratio_1m_1row_max"][0]
    long = traffic.dsa_bytes(1 << 20, score_bytes=0) / traffic.dense_mla_bytes(1 << 20)
    assert _close(long, g["ratio_long_context"])
    assert traffic.KEY_BYTES == g["key_bytes"][0] and traffic.LAT_BYTES == g["latent_bytes"][0]
    assert 24 * traffic.LAT_BYTES == g["kv_per_token_k3"][0]
    assert 24 * (traffic.LAT_BYTES + traffic.KEY_BYTES) == g["kv_per_token_k31"][0]


def test_counted_bytes_of_an_oracle_run_match_the_closed_form():
    case = make_case(1, 1, [12288], seed=15)
    res = oracle.dsa_rows(case)
    assert oracle.counted_bytes(case, res) == traffic.dsa_bytes(12288)
    case4 = make_case(2, 4, [3000, 5000], seed=16)
    res4 = oracle.dsa_rows(case4)
    pos = case4.positions().numpy()
    expect = 0
    for b, L in enumerate([3000, 5000]):
        expect += L * traffic.KEY_BYTES
        for r in range(4):
            n = int(pos[b * 4 + r]) + 1
            expect += min(2048, n) * traffic.LAT_BYTES + n * traffic.SCORE_BYTES
    assert oracle.counted_bytes(case4, res4) == expect
