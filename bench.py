"""Benchmark of the Step-5 sparse-indexer hot path on one MI355X.

A step is one decode pass of the whole path over a batch of rows, with every
input resident in HBM (each call captured once as a HIP graph and replayed,
so the step measures the GPU and not the Python launch path):
  1. step5_index_summarize   the region each row just completed (k prep +
                             summary, steps a2/a3)
  2. step5_index_score_topk  q prep, scores over all candidates, top 512 per
                             KV group (steps a1/a4/a5)
  3. step5_sparse_attn       attention over the picks plus the own region (a6)
The cache summaries of the whole context are built once before timing (one
step5_index_summarize over every token, itself timed and reported as the
summary phase).

Default workload: decode16_ctx128k (16 rows, each with its own 131,072-token
context, Student-t inputs). One JSON line goes to stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse-attn decode rows/s at 128K ctx; indexer HBM GB/s as % of peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode16_ctx128k")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2)
    ap.add_argument("--eager", action="store_true", help="launch the calls directly, no HIP graphs")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no sharding or collectives are built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_indexer_amd as s5
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.init()
    d = W.make_case(wl, args.seed, dev)
    rows, T, B = d["rows"], d["cache_tokens"], d["batch"]
    R_cap = T // 8
    eps = W.NORM_EPS
    scale = 1.0 / math.sqrt(W.HEAD_DIM)
    stream = torch.cuda.current_stream()

    # ---- one-time: summaries of the whole cache (also the summary-phase measurement)
    if wl.tie_heavy:
        S = d["summary"]
        sum_k, sum_z, sum_t0 = d["fresh_k"], d["fresh_z"], 0
        S_fresh = torch.zeros((1, wl.fresh_tokens // 8, 4, 64), dtype=torch.uint8, device=dev)
        full_pass = lambda: s5.step5_index_summarize(sum_k, sum_z, 0, d["ln_w"], d["ln_b"], eps,
                                                     d["rope"], S_fresh)
        full_tokens = wl.fresh_tokens
    else:
        S = torch.zeros((B, R_cap, 4, 64), dtype=torch.uint8, device=dev)
        full_pass = lambda: s5.step5_index_summarize(d["k_idx"], d["z_idx"], 0, d["ln_w"],
                                                     d["ln_b"], eps, d["rope"], S)
        full_tokens = B * T
    full_pass()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    ev0.record(stream)
    for _ in range(reps):
        full_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    summ_us = ev0.elapsed_time(ev1) * 1000.0 / reps
    summ_bytes = full_tokens * 1024 + (full_tokens // 8) * 256
    summ_gbs = summ_bytes / summ_us / 1e3

    # ---- the decode step
    p_last = T - 1
    own0 = (p_last // 8) * 8
    own_T = p_last + 1 - own0          # tokens of the own region present (8 at these workloads)
    ids = torch.empty((rows, 4, 512), dtype=torch.int32, device=dev)
    out = torch.empty((rows, 16, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=dev)
    ws1 = torch.empty(s5.step5_index_score_topk_workspace(rows, R_cap) + 256, dtype=torch.uint8,
                      device=dev)
    ws2 = torch.empty(max(1, s5.step5_sparse_attn_workspace(rows)) + 256, dtype=torch.uint8,
                      device=dev)
    ws1 = ws1[(-ws1.data_ptr()) % 256:]
    ws2 = ws2[(-ws2.data_ptr()) % 256:]
    if not wl.tie_heavy and own_T == 8 and not wl.prefill_chunk:
        k_own = d["k_idx"][:, own0:own0 + 8]
        z_own = d["z_idx"][:, own0:own0 + 8]
    else:
        k_own = z_own = None

    def call_summarize():
        if k_own is not None:
            s5.step5_index_summarize(k_own, z_own, own0, d["ln_w"], d["ln_b"], eps, d["rope"], S)

    def call_score():
        if wl.tie_heavy:
            s5.step5_index_score_topk(d["q8"], d["w_head"], d["row_seq"], d["row_pos"], S, ids,
                                      q_is_e4m3=True, workspace=ws1)
        else:
            s5.step5_index_score_topk(d["q_idx"], d["w_head"], d["row_seq"], d["row_pos"], S, ids,
                                      q_norm_w=d["q_norm_w"], q_eps=eps, rope=d["rope"],
                                      workspace=ws1)

    def call_attn():
        s5.step5_sparse_attn(d["q"], d["k_cache"], d["v_cache"], ids, d["row_seq"], d["row_pos"],
                             scale, out, lse, workspace=ws2)

    def call_indexer():
        # own-region summary (feeds the next step), then this step's selection
        call_summarize()
        call_score()

    calls = [("indexer", call_indexer), ("sparse_attn", call_attn)]
    for _ in range(args.warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    runners = dict(calls)
    if not args.eager:
        graphs = {}
        for name, f in calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            graphs[name] = g
        runners = {name: g.replay for name, g in graphs.items()}
        for _ in range(args.warmup):
            for name, _ in calls:
                runners[name]()
        torch.cuda.synchronize()
    nev = args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nev * (len(calls) + 1))]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        base = i * (len(calls) + 1)
        evs[base].record(stream)
        for c, (name, _) in enumerate(calls):
            runners[name]()
            evs[base + c + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call = {}
    for c, (name, _) in enumerate(calls):
        tot = 0.0
        for i in range(nev):
            base = i * (len(calls) + 1)
            tot += evs[base + c].elapsed_time(evs[base + c + 1])
        per_call[name] = tot * 1000.0 / nev
    ms_per_step = elapsed * 1000.0 / args.steps
    rows_per_s = rows * args.steps / elapsed

    # algorithmic bytes per launch
    nsel = min(512, p_last // 8)
    tok_per_unit = 8 * nsel + (p_last % 8) + 1
    attn_bytes = rows * 4 * tok_per_unit * 128 * 2 * 2
    score_bytes = rows * (p_last // 8) * 256
    own_bytes = (B * 8 * 1024 + B * 256) if k_own is not None else 0
    attn_gbs = attn_bytes / per_call["sparse_attn"] / 1e3
    score_gbs = score_bytes / per_call["indexer"] / 1e3

    result = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": rows, "context_tokens": T, "sequences": B,
                   "topk": 512, "region": 8, "idx_heads": 16, "kv_groups": 4, "q_heads": 16,
                   "head_dim": 128, "inputs": wl.dist},
        "roofline": {"bound": "hbm", "kernel": "step5_sparse_attn (attn_kernel + attn_merge_kernel)",
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": attn_bytes},
        "phases": {
            "graph_replay": not args.eager,
            "indexer_us": round(per_call["indexer"], 2),
            "sparse_attn_us": round(per_call["sparse_attn"], 2),
            "score_stream_GBs": round(score_gbs, 1),
            "score_stream_frac_hbm": round(score_gbs / HBM_PEAK_GBS, 4),
            "own_region_bytes": own_bytes,
            "summary_pass": {"tokens": full_tokens, "us": round(summ_us, 1),
                             "GBs": round(summ_gbs, 1),
                             "frac_hbm": round(summ_gbs / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes": summ_bytes},
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, wl, S, args.cpu_rows, torch)
    print(json.dumps(result), flush=True)


def cpu_baseline(d, wl, S_gpu, nrows, torch):
    """The oracle (unchanged) on a bounded sample of the same decode step: the
    first `nrows` rows, each over its own sequence. The oracle builds its own
    summaries of those sequences first (untimed, like the GPU's cache); then the
    timed part is the same step: own-region summary, q prep, scores, top-512
    selection and attention."""
    import numpy as np
    from oracle import oracle as orc
    import workloads as W

    nth = orc.default_threads()
    rows = list(range(min(nrows, d["rows"])))
    seqs = sorted({int(d["row_seq"][r]) for r in rows})
    smap = {s: i for i, s in enumerate(seqs)}
    T = d["cache_tokens"]
    rope = W.bits16(d["rope"])
    lnw, lnb = d["ln_w"].cpu().numpy(), d["ln_b"].cpu().numpy()
    if wl.tie_heavy:
        Sh = W.bits8(d["summary"][seqs])
    else:
        k16 = np.concatenate([W.bits16(d["k_idx"][s:s + 1]) for s in seqs])
        z16 = np.concatenate([W.bits16(d["z_idx"][s:s + 1]) for s in seqs])
        Sh = orc.summarize(k16, z16, 0, lnw, lnb, W.NORM_EPS, rope, nthreads=nth)
    kc = np.concatenate([W.bits16(d["k_cache"][s:s + 1]) for s in seqs])
    vc = np.concatenate([W.bits16(d["v_cache"][s:s + 1]) for s in seqs])
    pos = d["row_pos"].cpu().numpy()[rows]
    seq = np.array([smap[int(d["row_seq"][r])] for r in rows], np.int32)
    w = d["w_head"].cpu().numpy()
    q = W.bits16(d["q"])[rows]
    t0 = time.perf_counter()
    if not wl.tie_heavy:
        own0 = (T - 1) // 8 * 8
        orc.summarize(k16[:, own0:own0 + 8], z16[:, own0:own0 + 8], own0, lnw, lnb, W.NORM_EPS,
                      rope, R_cap=Sh.shape[1], summary=Sh, nthreads=nth)
        q8 = orc.q_prep(W.bits16(d["q_idx"])[rows], d["q_norm_w"].cpu().numpy(), W.NORM_EPS, rope,
                        pos, nthreads=nth)
    else:
        q8 = W.bits8(d["q8"])[rows]
    sc = orc.score(q8, w, seq, pos, Sh, nthreads=nth)
    ids, _ = orc.select(sc, pos, 512, nthreads=nth)
    orc.attend(q, kc, vc, ids, seq, pos, 1.0 / math.sqrt(W.HEAD_DIM), nthreads=nth)
    dt = time.perf_counter() - t0
    return {"value": round(len(rows) / dt, 3), "unit": "rows/s", "cores": nth, "kind": "oracle",
            "sample": f"{len(rows)} of {d['rows']} rows of {wl.name} (own-region summary, q prep, "
                      f"scores, top-512, attention); {dt:.2f} s"}


if __name__ == "__main__":
    main()
