"""Repeatability of the fused decode.

- Captured in a HIP graph (as the benchmark times it), every replay must give
  the eager result: the same selected set and attention within tolerance
  (outputs are cleared to NaN before each replay, so a write a replay missed
  shows). Replays alternate with eager work on the same workspace and use
  two input sets, so a captured launch that depended on state left by an
  earlier one would show as well.
- The selection's order is unspecified (it depends on the timing of LDS
  slot reservations), and attention sums in that order, so whole decodes
  agree to rounding only. Attention over one fixed selection must be
  bit-identical from call to call: a race in the attention kernel would
  break that.
"""

import pytest
import torch

import sparse_attention_index_amd as dsa
from tests.parity import check_attention
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=2, R=4, lengths=[3000, 5001], seed=801, permute_blocks=True),   # single-workgroup top-k
    dict(B=1, R=2, lengths=[50000], seed=802, permute_blocks=True),        # slice + final top-k
]


def _run(case, batch, cache, ws, out, lse, idx):
    dsa.dsa_decode(batch, cache, case.q_idx, case.w, case.q_mla, case.topk, case.sm_scale, out, lse, idx, ws,
                   q_scale=case.q_idx_scale)


def _check(tag, got, ref):
    o, l, i = got
    assert not torch.isnan(o.float()).any() and not torch.isnan(l).any(), f"{tag}: unwritten outputs"
    assert torch.equal(i.sort(dim=1).values, ref[2]), f"{tag}: selection"
    check_attention(o.float().cpu().numpy(), l.cpu().numpy(), ref[0].float().cpu().numpy(), ref[1].cpu().numpy(), tag)


@pytest.mark.parametrize("kw", CASES, ids=["2x4_short_topk", "1x2_long_topk"])
def test_graph_replays_equal_eager(gpu, kw):
    print(f"\n[case] graph {kw}", flush=True)
    cases = [make_case(name="graph", **dict(kw, seed=kw["seed"] + 10 * i)).to("cuda") for i in range(2)]
    rows, k = cases[0].rows, cases[0].topk
    max_ctx = max(c.max_ctx for c in cases)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, rows, max_ctx, k))
    bufs = [(torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda"),
             torch.empty((rows, 16), dtype=torch.float32, device="cuda"),
             torch.empty((rows, k), dtype=torch.int32, device="cuda")) for _ in cases]
    batches = [dsa.Batch.of(c) for c in cases]
    caches = [dsa.Cache.of(c) for c in cases]

    ref = []
    for c, b, ch, (o, l, i) in zip(cases, batches, caches, bufs):
        _run(c, b, ch, ws, o, l, i)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone(), i.sort(dim=1).values))

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c, b, ch, (o, l, i) in zip(cases, batches, caches, bufs):
            _run(c, b, ch, ws, o, l, i)
    torch.cuda.synchronize()

    for rep in range(4):
        for o, l, i in bufs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
            i.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for j, got in enumerate(bufs):
            _check(f"replay {rep} set {j}", got, ref[j])
        # eager work on the same workspace between replays
        j = rep % 2
        _run(cases[j], batches[j], caches[j], ws, *bufs[j])
        torch.cuda.synchronize()
        _check(f"eager after replay {rep} set {j}", bufs[j], ref[j])


def test_attention_on_a_fixed_selection_is_bit_identical(gpu):
    case = make_case(name="repeat", B=2, R=4, lengths=[3000, 5001], seed=803, permute_blocks=True).to("cuda")
    print("\n[case] repeat 2x4", flush=True)
    rows, k = case.rows, case.topk
    b, c = dsa.Batch.of(case), dsa.Cache.of(case)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, rows, case.max_ctx, k))
    sel = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    _run(case, b, c, ws, torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda"),
         torch.empty((rows, 16), dtype=torch.float32, device="cuda"), sel)
    mws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_MLA_DECODE, rows, 0, k))
    first = None
    for call in range(5):
        o = torch.full((rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        l = torch.full((rows, 16), float("nan"), dtype=torch.float32, device="cuda")
        dsa.dsa_sparse_mla_decode(b, c, case.q_mla, sel, case.sm_scale, o, l, mws)
        torch.cuda.synchronize()
        if first is None:
            first = (o, l)
        else:
            assert torch.equal(o.view(torch.int16), first[0].view(torch.int16)), f"call {call}: out"
            assert torch.equal(l.view(torch.int32), first[1].view(torch.int32)), f"call {call}: lse"
