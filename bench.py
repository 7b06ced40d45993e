#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

A step is one pass of the whole hot path -- Score (lightning indexer over
every cached FP8 key), Select (exact top-2048 per query row) and Attend
(sparse MLA over the selected latent rows) -- through the fused dsa_decode
entry point. The default batch is the largest decode configuration: 4
requests x 4 verification rows at 1,048,576 tokens of context each, with
about 1% of the keys planted along the query direction (+3 sigma). Inputs
are seeded synthetic tensors resident in HBM; independent input sets are
rotated so that successive steps do not hit in the 256 MB Infinity Cache.

Prints one JSON line. `value` is context tokens scanned per second (the sum
of the requests' context lengths per step over the step time); rows/s, the
whole-step HBM fraction, per-stage times (each stage's entry point in step
order, its launches bracketed by events), the roofline of the dominant kernel
(the scorer the step runs, timed as its stage) and a float64 CPU oracle
baseline are added beside it. Past 40,960 tokens the step takes the filtered
path (the scorer keeps only candidates at or above a sampled threshold), and
the stages are that path's.

`--workload prefill_4096_on_128k` measures a prefill chunk instead (FP8-query
indexer over the causal history, per-row top-k, sparse MLA prefill) and reports
the scorer against the FP8 MFMA peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
MALL_BYTES = 256 << 20
# dsa_decode filters the scores of batches with max_ctx above FILTER_MIN_CTX
# (csrc/api.hip); the top-k selects rows of at most SHORT_TOPK_MAX scores in
# one workgroup each (csrc/topk.hip)
FILTER_MIN_CTX = 40960
SHORT_TOPK_MAX = 40960


def _b(x):
    return str(bool(x)).lower()


def sample_kernels(rows, R, mxfp4, q_fp8=False):
    """The sampling pass's two kernels as profiles name them: 128 sampled pages per row up to 32
    rows, 64 beyond; past 8 rows per request the many-rows kernel (filter.hip)."""
    nsp = 128 if rows <= 32 else 64
    if R > 8:
        return [f"sample_score_rows_kernel<{_b(mxfp4)},{nsp},{_b(q_fp8)}>", "sample_select_kernel"]
    return [f"sample_score_kernel<{_b(mxfp4)},{nsp},2,{_b(q_fp8)}>", "sample_select_kernel"]


def score_rpw(R, q_fp8=False):
    """Query rows per wave of the scorer variant a row group of R rows takes (csrc/score.hip)."""
    if q_fp8:
        return 4 if R > 16 else 2 if R > 4 else 1
    return 2 if R > 4 else 1
METRIC = "DSA decode: context tokens scanned/s + query rows/s; % of HBM roofline"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_4x4_1m_planted")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to exceed 3x the MALL)")
    ap.add_argument("--eager", action="store_true", help="launch every step from the host instead of a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle baseline (0: skip)")
    return ap.parse_args()


def _code_only(text):
    """Source text without comments and whitespace (string literals kept), so
    that only a change to the code itself changes the hash."""
    text = re.sub(r'"(?:\\.|[^"\\])*"|/\*.*?\*/|//[^\n]*',
                  lambda m: m.group(0) if m.group(0).startswith('"') else " ", text, flags=re.S)
    return re.sub(r"\s+", "", text)


def kernel_source_hash(name):
    """Hash of the code of a kernel's source file and of every header beside it (what it may include)."""
    csrc = os.path.join(ROOT, "sparse_attention_index_amd", "csrc")
    h = hashlib.sha256()
    for n in [name] + sorted(f for f in os.listdir(csrc) if f.endswith(".h")):
        with open(os.path.join(csrc, n), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _counter_lines(workload):
    path = os.path.join(ROOT, "profiles", "hbm_counters.txt")
    if not os.path.exists(path):
        return []
    with open(path) as f:
        return [p for p in (line.split() for line in f if not line.startswith("#")) if len(p) == 6 and p[1] == workload]


def counters_for(kernel, workload):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter summary.

    profiles/hbm_counters.txt holds one line per (kernel, workload):
    `<file> <workload> <kernel> <source hash> <fetch bytes> <write bytes>` (already scaled by
    the copy-kernel calibration). The entry counts only while the kernel's sources are unchanged.
    """
    for p in _counter_lines(workload):
        if p[2] == kernel:
            return float(p[4]) + float(p[5]) if p[3] == kernel_source_hash(p[0]) else None
    return None


def measured_step_bytes(workload, kernels):
    """HBM bytes of one whole step as rocprofv3 counted them: the sum over the
    step's kernels, or None if one is missing or its sources have changed since."""
    got = {p[2]: p for p in _counter_lines(workload)}
    total = 0.0
    for kname in kernels:
        p = got.get(kname)
        if p is None or p[3] != kernel_source_hash(p[0]):
            return None
        total += float(p[4]) + float(p[5])
    return total


def _blas_threads():
    """Threads of numpy's BLAS pool (the oracle's matrix products run there)."""
    try:
        from threadpoolctl import threadpool_info

        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


def _host_cores():
    """Cores this process may run on (its CPU affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _cores_fields():
    # the oracle is numpy: its matrix products use the BLAS pool, the rest one thread
    return {"cores": min(_host_cores(), _blas_threads()), "host_cores": _host_cores(),
            "blas_threads": _blas_threads()}


def cpu_baseline(workload_name, budget_s):
    """The float64 oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    from workloads import case_config, make_case, structure_kwargs

    cfg = case_config(workload_name)
    R, lens = cfg["R"], cfg["lengths"]
    kw = structure_kwargs(cfg)
    if R > 64:  # prefill chunk: one request, sample its query rows
        case = make_case(1, R, lens[:1], seed=cfg["seed"] + 1000, **kw)
        rows, spent = 0, 0.0
        step = max(1, R // 64)
        while rows < R and (spent < budget_s or rows == 0):
            t0 = time.perf_counter()
            oracle.dsa_rows(case, rows=[(rows * step) % R])
            spent += time.perf_counter() - t0
            rows += 1
        return {"value": rows / spent, "unit": "rows/s", **_cores_fields(), "kind": "oracle",
                "sample": f"{rows} of {R} query rows (spread over the chunk) of a re-seeded chunk of the same "
                          f"shape and structure, all stages, numpy float64 on the host, {spent:.1f} s"}
    done, tokens, rows, spent = 0, 0, 0, 0.0
    while done < len(lens) and (spent < budget_s or done == 0):
        case = make_case(1, R, [lens[done]], seed=cfg["seed"] + 1000 + done, **kw)
        t0 = time.perf_counter()
        oracle.dsa_rows(case)
        spent += time.perf_counter() - t0
        tokens += lens[done]
        rows += R
        done += 1
    return {
        "value": tokens / spent,
        "unit": "tokens/s",
        "rows_per_s": rows / spent,
        **_cores_fields(),
        "kind": "oracle",
        "sample": f"{done} of {len(lens)} requests ({rows} rows, context {lens[:done]}), each re-seeded with "
                  f"the workload's shape and structure, all stages, numpy float64 on the host, {spent:.1f} s",
    }


def kernel_time(torch, fn, nsets, n=20):
    """Average launch time of a one-kernel entry point: n launches back to back on the current
    stream (rotating over the input sets) between two events. A GPU-side sleep ahead of them
    lets the host enqueue all n first, so no host gap falls inside the timed span. Stream order
    serialises the launches, as inside the decode step."""
    fn(0)  # untimed
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e8))
    ev0.record()
    for i in range(n):
        fn(i % nsets)
    ev1.record()
    torch.cuda.synchronize()
    return 1e3 * ev0.elapsed_time(ev1) / n


def stage_times(torch, stages, n):
    """Per-stage event times when the stages run in order, repeated n times."""
    evs = {s: [] for s, _ in stages}
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for i in range(n):
        for s, fn in stages:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(i)
            e1.record()
            evs[s].append((e0, e1))
    torch.cuda.synchronize()
    return {s: 1e3 * sum(a.elapsed_time(b) for a, b in v) / n for s, v in evs.items()}


def step_hbm_fields(traffic, lens, R, k, kfmt, sec, workload, kernels, filtered):
    """The step's algorithmic bytes over its time (keys once, selected latents,
    and on the stored-score path the fp32 score round trip); the same without
    that round trip; and the rocprofv3-counted bytes of the step's kernels
    over the same time."""
    step_bytes = traffic.decode_step_bytes(lens, R, k, kfmt, round_trip=not filtered)
    no_rt = traffic.decode_step_bytes(lens, R, k, kfmt, round_trip=False)
    meas = measured_step_bytes(workload, kernels)
    return {
        "path": "filtered" if filtered else "stored scores",
        "bytes": step_bytes,
        "achieved_GBs": step_bytes / sec / 1e9,
        "frac": step_bytes / sec / 1e9 / HBM_PEAK_GBS,
        "frac_without_score_round_trip": no_rt / sec / 1e9 / HBM_PEAK_GBS,
        "measured_bytes": meas,
        "measured_frac": None if meas is None else meas / sec / 1e9 / HBM_PEAK_GBS,
    }


def run_decode(args, torch, dsa, traffic, cfg):
    from workloads import make_case, structure_kwargs

    B, R, lens = cfg["B"], cfg["R"], cfg["lengths"]
    k = 2048
    rows = B * R
    kfmt = cfg.get("key_format", "fp8")
    q_fp8 = bool(cfg.get("fp8_query", False))  # E4M3 index queries with row scales
    step_bytes = traffic.decode_step_bytes(lens, R, k, kfmt)
    filtered = max(lens) > FILTER_MIN_CTX
    set_bytes = sum(lens) * (traffic.key_bytes(kfmt) + traffic.LAT_ROW_BYTES)
    nsets = args.sets or max(2, math.ceil(3 * MALL_BYTES / min(step_bytes, set_bytes)))
    nsets = min(nsets, max(2, int(40e9 // set_bytes)))

    kw = structure_kwargs(cfg)
    cases = [make_case(B, R, lens, seed=cfg["seed"] + 100 * i, device="cuda", name=args.workload, **kw)
             for i in range(nsets)]
    batches = [dsa.Batch.of(c) for c in cases]
    caches = [dsa.Cache.of(c) for c in cases]
    max_ctx = max(lens)
    ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_DECODE, rows, max_ctx, k))
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, 16), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")

    def step(i):
        c = cases[i]
        dsa.dsa_decode(batches[i], caches[i], c.q_idx, c.w, c.q_mla, k, c.sm_scale, out, lse, idx, ws,
                       q_scale=c.q_idx_scale)

    for i in range(args.warmup):
        step(i % nsets)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(nsets):
                step(i)
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps
    reps = math.ceil(args.steps / nsets) if graph is not None else 0
    steps_run = reps * nsets if graph is not None else args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    if graph is not None:
        for _ in range(reps):
            graph.replay()
    else:
        for i in range(steps_run):
            step(i % nsets)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / steps_run

    # ---- stage-wise entry points on the same inputs
    ld = (max_ctx + 63) // 64 * 64
    scores = torch.empty((rows, ld), dtype=torch.float32, device="cuda")
    row_len = [(c.positions() + 1).to(torch.int32).cuda() for c in cases]
    tk_ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, rows, ld, k))
    mla_ws_n = dsa.dsa_workspace_size(dsa.DSA_WS_MLA_DECODE, rows, 0, k)
    mla_ws = dsa.workspace(mla_ws_n) if mla_ws_n else None
    n_stage = min(args.steps, 100)

    def score(i):
        j = i % nsets
        dsa.dsa_index_score(batches[j], caches[j], cases[j].q_idx, cases[j].w, scores, q_scale=cases[j].q_idx_scale)

    def topk(i):
        dsa.dsa_topk(scores, row_len[i % nsets], k, idx, tk_ws)

    def attend(i):
        j = i % nsets
        dsa.dsa_sparse_mla_decode(batches[j], caches[j], cases[j].q_mla, idx, cases[j].sm_scale, out, lse, mla_ws)

    stored = stage_times(torch, [("score", score), ("topk", topk), ("attend", attend)], n_stage)
    if filtered:
        # the filtered path's stages, one workspace per input set (each keeps
        # its own thresholds and candidates from one stage to the next)
        wss = [ws] + [dsa.workspace(ws.numel()) for _ in range(nsets - 1)]

        def f_thr(i):
            j = i % nsets
            dsa.dsa_filter_threshold(batches[j], caches[j], cases[j].q_idx, cases[j].w, k, wss[j],
                                     q_scale=cases[j].q_idx_scale)

        def f_score(i):
            j = i % nsets
            dsa.dsa_filter_score(batches[j], caches[j], cases[j].q_idx, cases[j].w, k, wss[j],
                                 q_scale=cases[j].q_idx_scale)

        def f_select(i):
            j = i % nsets
            dsa.dsa_filter_select(batches[j], caches[j], cases[j].q_idx, cases[j].w, k, idx, wss[j],
                                  q_scale=cases[j].q_idx_scale)

        stage_us = stage_times(torch, [("threshold", f_thr), ("score", f_score), ("select", f_select),
                                       ("attend", attend)], n_stage)
        stage_us["stored_path"] = {"score": stored["score"], "topk": stored["topk"]}
        # ---- dominant kernel: the filtered scorer, one kernel per dsa_filter_score call,
        # timed inside the stage sequence above
        score_us = stage_us["score"]
        dom_bytes = traffic.filter_scorer_bytes(lens, R, kfmt, q_fp8)
        dom_kernel = f"score_kernel<{score_rpw(R)},{_b(q_fp8)},{_b(kfmt == 'mxfp4')},true>"
        step_kernels = sample_kernels(len(lens) * R, R, kfmt == "mxfp4", q_fp8) + [
            dom_kernel, f"candidate_select_kernel<{_b(kfmt == 'mxfp4')},{_b(q_fp8)}>"]
    else:
        stage_us = stored
        # ---- dominant kernel: the indexer scorer (its share of the step grows with context),
        # one kernel per dsa_index_score call, timed inside the stage sequence above
        score_us = stage_us["score"]
        dom_bytes = traffic.scorer_bytes(lens, R, kfmt, q_fp8)
        dom_kernel = f"score_kernel<{score_rpw(R, q_fp8)},{_b(q_fp8)},{_b(kfmt == 'mxfp4')},false>"
        step_kernels = [dom_kernel, "topk_short_kernel<true>" if max_ctx <= SHORT_TOPK_MAX else "topk_slice_kernel<true>"]
        if max_ctx > SHORT_TOPK_MAX:
            step_kernels.append("topk_final_kernel<true>")
    step_kernels += ["sparse_mla_kernel"] + (["mla_combine_kernel"] if mla_ws_n else [])
    achieved = dom_bytes / (score_us * 1e-6) / 1e9

    tokens = sum(lens)
    sec = ms_step * 1e-3
    return {
        "metric": METRIC,
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_run,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if q_fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "requests": B,
            "rows_per_request": R,
            "context": lens[0] if len(set(lens)) == 1 else [min(lens), max(lens)],
            "topk": k,
            "indexer": ("32h x 128d, MXFP4 keys (E2M1 + E8M0 per 32 dims, 68 B)" if kfmt == "mxfp4"
                        else "32h x 128d, E4M3 keys + fp32 scale")
            + (", E4M3 queries + fp32 row scale" if q_fp8 else ", bf16 queries"),
            "mla": "16h x 576 latent (E4M3 + fp32 scale) -> 512",
            "input_sets_rotated": nsets,
            "launch": "eager" if graph is None else "hip graph",
        },
        "rows_per_s": rows / sec,
        "step_hbm": step_hbm_fields(traffic, lens, R, k, kfmt, sec, args.workload, step_kernels, filtered),
        "stages_us": stage_us,
        "wall_s": wall,
        "roofline": {
            "bound": "hbm",
            "kernel": dom_kernel,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counters_for(dom_kernel, args.workload),
            "algorithmic_bytes": dom_bytes,
            "avg_launch_us": score_us,
        },
    }


def run_prefill(args, torch, dsa, traffic, cfg):
    """Prefill chunk: FP8-query indexer over the whole causal history, per-row top-k, sparse MLA."""
    from workloads import make_case, structure_kwargs

    R, L = cfg["R"], cfg["lengths"][0]
    k = 2048
    kw = structure_kwargs(cfg)
    case = make_case(1, R, [L], seed=cfg["seed"], device="cuda", name=args.workload, **kw)
    batch, cache = dsa.Batch.of(case), dsa.Cache.of(case)
    ld = (L + 63) // 64 * 64
    scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    row_len = (case.positions() + 1).to(torch.int32).cuda()
    tk_ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, R, ld, k))
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    out = torch.empty((R, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, 16), dtype=torch.float32, device="cuda")

    def score(i):
        dsa.dsa_index_score(batch, cache, case.q_idx, case.w, scores, q_scale=case.q_idx_scale)

    def topk(i):
        dsa.dsa_topk(scores, row_len, k, idx, tk_ws)

    def attend(i):
        dsa.dsa_sparse_mla_prefill(batch, cache, case.q_mla, idx, case.sm_scale, out, lse)

    def step(i):
        score(i)
        topk(i)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    n_stage = min(args.steps, 10)
    stage_us = stage_times(torch, [("score", score), ("topk", topk), ("attend", attend)], n_stage)
    score_us = kernel_time(torch, score, 1)
    flops = traffic.scorer_flops([L], R)
    tflops = flops / (score_us * 1e-6) / 1e12
    sec = ms_step * 1e-3
    return {
        "metric": "DSA prefill chunk: query rows/s; indexer % of FP8 MFMA roofline",
        "value": R / sec,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": R, "history": L - R, "keys": L, "topk": k,
                   "indexer": "FP8 q (row scale) x E4M3 keys, 32h x 128d", "mla": "16h x 576 -> 512"},
        "context_tokens_per_s": L / sec,
        "stages_us": stage_us,
        "wall_s": wall,
        "roofline": {
            "bound": "mfma",
            "kernel": f"score_kernel<{score_rpw(R, True)},true,false,false>",
            "achieved": tflops,
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / FP8_PEAK_TFLOPS,
            "traffic": counters_for(f"score_kernel<{score_rpw(R, True)},true,false,false>", args.workload),
            "algorithmic_flops": flops,
            "avg_launch_us": score_us,
        },
    }


KEY_WRITE = {
    # name: (requests, new rows per request, context of each request)
    "index_key_write_4096": (1, 4096, 135168),   # the prefill chunk's new keys
    "index_key_write_16x4": (16, 4, 32768),      # one decode step's new keys
}
KEY_WRITE_ROW_BYTES = 256 + 128 + 4 + 4  # bf16 key in, E4M3 codes + scale out, page id


def run_key_write(args, torch, dsa):
    """The index-key write step alone: LayerNorm + E4M3 absmax quantisation +
    paged write of every new row's key (device-resident inputs)."""
    B, R, L = KEY_WRITE[args.workload]
    nb = B * ((L + 63) // 64)
    g = torch.Generator(device="cuda")
    g.manual_seed(20260100)
    ctx = torch.full((B,), L, dtype=torch.int32, device="cuda")
    table = torch.randperm(nb, generator=g, device="cuda").to(torch.int32).reshape(B, -1)
    batch = dsa.Batch(R, ctx, table, L)
    nsets = 4
    ks = [torch.randn((B * R, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(nsets)]
    w = (1.0 + 0.1 * torch.randn(128, generator=g, device="cuda")).float()
    b = (0.1 * torch.randn(128, generator=g, device="cuda")).float()
    key_fp8 = torch.zeros((nb, 64, 128), dtype=torch.uint8, device="cuda")
    key_scale = torch.ones((nb, 64), dtype=torch.float32, device="cuda")

    def step(i):
        dsa.dsa_index_key_write(batch, ks[i % nsets], w, b, key_fp8, key_scale)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(1e8))  # the host queues every launch before the GPU reaches them
    ev0.record()
    for i in range(n):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    us = 1e3 * ev0.elapsed_time(ev1) / n
    rows = B * R
    achieved = rows * KEY_WRITE_ROW_BYTES / (us * 1e-6) / 1e9
    return {
        "metric": "DSA index-key write: new rows/s; % of HBM roofline",
        "value": rows / (us * 1e-6),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "requests": B, "rows_per_request": R, "context": L,
                   "launch": "eager, back to back"},
        "roofline": {
            "bound": "hbm",
            "kernel": "index_key_write_kernel",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes": rows * KEY_WRITE_ROW_BYTES,
            "avg_launch_us": us,
        },
    }


DCP = {
    # name: (decode workload, virtual shards W)
    "dcp8_decode_16x4_32k": ("decode_16x4_32k", 8),
    "dcp8_decode_16x4_ragged_128k_256k": ("decode_16x4_ragged_128k_256k", 8),
}


def run_dcp(args, torch, dsa, traffic):
    """One decode step under decode context parallelism, simulated on this
    GPU: score -> exact top-k merge over W virtual shards -> per-shard sparse
    MLA + LSE combine. The shards are regions of one device's memory, so this
    measures the merge's and the combine's device work, not the exchanges."""
    from workloads import case_config, make_case, structure_kwargs

    base, W = DCP[args.workload]
    cfg = case_config(base)
    B, R, lens = cfg["B"], cfg["R"], cfg["lengths"]
    k, C = 2048, int(1.5 * 2048 / W)
    rows = B * R
    kw = structure_kwargs(cfg)
    nsets = 2
    cases = [make_case(B, R, lens, seed=cfg["seed"] + 100 * i, device="cuda", name=base, **kw) for i in range(nsets)]
    batches = [dsa.Batch.of(c) for c in cases]
    caches = [dsa.Cache.of(c) for c in cases]
    row_len = [(c.positions() + 1).to(torch.int32).cuda() for c in cases]
    ld = (max(lens) + 63) // 64 * 64
    scores = torch.empty((rows, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    resend = torch.empty((rows, W), dtype=torch.uint8, device="cuda")
    out = torch.empty((rows, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, 16), dtype=torch.float32, device="cuda")
    tws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_TOPK, rows, ld, k, W, C))
    mws = dsa.workspace(dsa.dsa_dcp_workspace_size(dsa.DSA_WS_DCP_MLA, rows, 0, k, W))

    def score(i):
        j = i % nsets
        dsa.dsa_index_score(batches[j], caches[j], cases[j].q_idx, cases[j].w, scores, q_scale=cases[j].q_idx_scale)

    def merge(i):
        dsa.dsa_dcp_topk(scores, row_len[i % nsets], k, W, C, idx, resend, tws)

    def attend(i):
        j = i % nsets
        dsa.dsa_dcp_mla_decode(batches[j], caches[j], cases[j].q_mla, idx, W, cases[j].sm_scale, out, lse, mws)

    def step(i):
        score(i)
        merge(i)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(1e8))
    ev0.record()
    for i in range(n):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / n
    stage_us = stage_times(torch, [("score", score), ("dcp_topk", merge), ("dcp_attend", attend)], min(n, 50))
    # the merge stage against HBM: its algorithmic input is every visible score, read once
    merge_us = kernel_time(torch, merge, nsets)
    vis = sum(traffic.visible(lens, R))
    merge_bytes = vis * traffic.SCORE_BYTES + rows * k * 4
    achieved = merge_bytes / (merge_us * 1e-6) / 1e9
    sec = ms_step * 1e-3
    return {
        "metric": METRIC,
        "value": sum(lens) / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "decode_workload": base, "virtual_shards": W, "candidates": C,
                   "requests": B, "rows_per_request": R, "topk": k,
                   "note": "DCP simulated on one GPU: merge and LSE combine on device, no exchange",
                   "launch": "eager, back to back"},
        "rows_per_s": rows / sec,
        "stages_us": stage_us,
        "resend_rows": int(resend.any(dim=1).sum().item()),
        "roofline": {
            "bound": "hbm",
            "kernel": "dcp_topk (stage)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes": merge_bytes,
            "avg_launch_us": merge_us,
        },
    }


def dcp_cpu_baseline(workload_name, budget_s):
    """The oracle's DCP merge on random score rows of the workload's length."""
    import numpy as np

    import oracle
    from workloads import case_config

    base, W = DCP[workload_name]
    cfg = case_config(base)
    L = cfg["lengths"][0]
    rng = np.random.default_rng(2)
    rows, spent = 0, 0.0
    while spent < budget_s or rows == 0:
        s = rng.standard_normal(L)
        t0 = time.perf_counter()
        oracle.dcp_select(s, W, 2048)
        spent += time.perf_counter() - t0
        rows += 1
        if rows >= 200:
            break
    return {"value": rows * L / spent, "unit": "tokens/s", "rows_per_s": rows / spent, **_cores_fields(),
            "kind": "oracle",
            "sample": f"{rows} score rows of {L} tokens, merge only (W = {W}), numpy on the host, {spent:.1f} s"}


def key_write_cpu_baseline(workload_name, budget_s):
    """The oracle's key write on the same number of rows (host numpy)."""
    import numpy as np

    import oracle

    B, R, L = KEY_WRITE[workload_name]
    rng = np.random.default_rng(1)
    k = rng.standard_normal((B * R, 128)).astype(np.float32)
    w, b = np.ones(128), np.zeros(128)
    reps, spent = 0, 0.0
    while spent < budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.index_key_write(k, w, b, 1e-6)
        spent += time.perf_counter() - t0
        reps += 1
        if reps >= 50:
            break
    return {"value": reps * B * R / spent, "unit": "rows/s", **_cores_fields(), "kind": "oracle",
            "sample": f"{reps} x {B * R} rows, LayerNorm + quantisation, numpy on the host, {spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the DSA path here has no "
              "multi-GPU mode. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_index_amd as dsa
    from sparse_attention_index_amd import traffic
    from workloads import case_config

    dsa.load()
    torch.cuda.set_device(0)
    if args.workload in DCP:
        result = run_dcp(args, torch, dsa, traffic)
        if args.cpu_seconds > 0:
            result["cpu_baseline"] = dcp_cpu_baseline(args.workload, min(args.cpu_seconds, 15.0))
        print(json.dumps(result), flush=True)
        return
    if args.workload in KEY_WRITE:
        result = run_key_write(args, torch, dsa)
        if args.cpu_seconds > 0:
            result["cpu_baseline"] = key_write_cpu_baseline(args.workload, min(args.cpu_seconds, 5.0))
        print(json.dumps(result), flush=True)
        return
    cfg = case_config(args.workload)
    if cfg["R"] > 64:
        result = run_prefill(args, torch, dsa, traffic, cfg)
    else:
        result = run_decode(args, torch, dsa, traffic, cfg)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
