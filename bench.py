#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

A step is one pass of the whole hot path -- Score (lightning indexer over
every cached FP8 key), Select (exact top-2048 per query row) and Attend
(sparse MLA over the selected latent rows) -- for one batch of 16 requests x
4 verification rows at 32,768 tokens of context each, through the fused
dsa_decode entry point. Inputs are seeded synthetic tensors resident in HBM;
several independent input sets are rotated so that successive steps do not
hit in the 256 MB Infinity Cache.

Prints one JSON line. `value` is context tokens scanned per second (the sum
of the requests' context lengths per step over the step time); rows/s, the
whole-step HBM fraction, per-stage times, the dominant kernel's roofline and a
float64 CPU oracle baseline are added beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "DSA decode: context tokens scanned/s + query rows/s; % of HBM roofline"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_16x4_32k")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to exceed 3x the MALL)")
    ap.add_argument("--eager", action="store_true", help="launch every step from the host instead of a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle baseline (0: skip)")
    return ap.parse_args()


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_index_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_for(kernel_file, workload):
    """HBM traffic measured by rocprofv3 counters for this kernel source, if current."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(f"{kernel_file}:{workload}")
    if not entry or entry.get("source_hash") != kernel_source_hash([kernel_file, "common.h"]):
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(workload_name, budget_s):
    """The float64 oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np  # noqa: F401

    import oracle
    from workloads import case_config, make_case

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cfg = case_config(workload_name)
    R, lens = cfg["R"], cfg["lengths"]
    done, tokens, rows, spent = 0, 0, 0, 0.0
    while done < len(lens) and (spent < budget_s or done == 0):
        case = make_case(1, R, [lens[done]], seed=cfg["seed"] + 1000 + done,
                         permute_blocks=cfg.get("permute_blocks", False),
                         plant_frac=cfg.get("plant_frac", 0.0), fp8_query=cfg.get("fp8_query", False))
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
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(lens)} requests ({rows} rows, context {lens[0]}), all stages, "
                  f"numpy float64 on the host, {spent:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the DSA path here has no "
              "multi-GPU mode. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_index_amd as dsa
    from sparse_attention_index_amd import traffic
    from workloads import case_config, make_case

    dsa.load()
    torch.cuda.set_device(0)
    cfg = case_config(args.workload)
    B, R, lens = cfg["B"], cfg["R"], cfg["lengths"]
    k = 2048
    rows = B * R
    step_bytes = traffic.decode_step_bytes(lens, R, k)
    set_bytes = sum(lens) * (traffic.KEY_BYTES + traffic.LAT_ROW_BYTES)
    nsets = args.sets or max(2, math.ceil(3 * MALL_BYTES / min(step_bytes, set_bytes)))
    nsets = min(nsets, max(2, int(40e9 // set_bytes)))

    kw = {k_: v for k_, v in cfg.items() if k_ in ("permute_blocks", "plant_frac", "fp8_query")}
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
        dsa.dsa_decode(batches[i], caches[i], c.q_idx, c.w, c.q_mla, k, c.sm_scale, out, lse, idx, ws)

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

    # ---- per-stage kernel times (stage-wise entry points, same inputs, host kept ahead of the GPU)
    ld = (max_ctx + 63) // 64 * 64
    scores = torch.empty((rows, ld), dtype=torch.float32, device="cuda")
    row_len = [(c.positions() + 1).to(torch.int32).cuda() for c in cases]
    tk_ws = dsa.workspace(dsa.dsa_workspace_size(dsa.DSA_WS_TOPK, rows, ld, k))
    mla_ws_n = dsa.dsa_workspace_size(dsa.DSA_WS_MLA_DECODE, rows, 0, k)
    mla_ws = dsa.workspace(mla_ws_n) if mla_ws_n else None
    n_stage = min(args.steps, 100)
    names = ("score", "topk", "attend")
    evs = {s: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_stage)]
           for s in names}
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))  # keep the GPU busy while the host enqueues every stage call
    for i in range(n_stage):
        c, j = cases[i % nsets], i % nsets
        e = evs["score"][i]
        e[0].record()
        dsa.dsa_index_score(batches[j], caches[j], c.q_idx, c.w, scores)
        e[1].record()
        e = evs["topk"][i]
        e[0].record()
        dsa.dsa_topk(scores, row_len[j], k, idx, tk_ws)
        e[1].record()
        e = evs["attend"][i]
        e[0].record()
        dsa.dsa_sparse_mla_decode(batches[j], caches[j], c.q_mla, idx, c.sm_scale, out, lse, mla_ws)
        e[1].record()
    torch.cuda.synchronize()
    stage_us = {s: 1e3 * sum(a.elapsed_time(b) for a, b in evs[s]) / n_stage for s in names}

    # ---- dominant kernel roofline: the indexer scorer (one kernel per call) or sparse MLA
    alg = {
        "score": (traffic.scorer_bytes(lens, R), "score.hip", "score_kernel"),
        "attend": (traffic.mla_bytes(lens, R, k), "mla.hip", "sparse_mla_kernel"),
    }
    dom = max(("score", "attend"), key=lambda s: stage_us[s])
    dom_bytes, dom_file, dom_kernel = alg[dom]
    achieved = dom_bytes / (stage_us[dom] * 1e-6) / 1e9
    measured = counters_for(dom_file, args.workload)

    tokens = sum(lens)
    sec = ms_step * 1e-3
    result = {
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "requests": B,
            "rows_per_request": R,
            "context": lens[0] if len(set(lens)) == 1 else [min(lens), max(lens)],
            "topk": k,
            "indexer": "32h x 128d, E4M3 keys + fp32 scale",
            "mla": "16h x 576 latent (E4M3 + fp32 scale) -> 512",
            "input_sets_rotated": nsets,
            "launch": "eager" if graph is None else "hip graph",
        },
        "rows_per_s": rows / sec,
        "step_hbm": {"bytes": step_bytes, "achieved_GBs": step_bytes / sec / 1e9,
                     "frac": step_bytes / sec / 1e9 / HBM_PEAK_GBS},
        "stages_us": stage_us,
        "wall_s": wall,
        "roofline": {
            "bound": "hbm",
            "kernel": dom_kernel,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured,
            "algorithmic_bytes": dom_bytes,
            "avg_launch_us": stage_us[dom],
        },
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
