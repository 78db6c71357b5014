"""Benchmark of the Step-5 sparse-indexer hot path on one MI355X.

A step is one pass of the whole path over a batch of rows of one attention
layer, with every input resident in HBM (the calls captured as HIP graphs and
replayed, so the step measures the GPU and not the Python launch path; one
graph holds one step per layer copy, as a decode pass captures all of a
model's layers, and the one-graph-per-step figure is reported beside it):
  1. step5_index_append      decode: each row's new token into the k/z rings and
                             the region it completes summarised (prefill:
                             step5_index_summarize over the chunk)
  2. step5_index_score_topk  q prep, scores over all candidates, top 512 per
                             KV group
     (decode rows of distinct sequences: 1 and 2 as one call,
     step5_index_append_score_topk, the appends in the selection's launch)
  3. step5_sparse_attn       attention over the picks plus the own region
The summaries of the context before the step are built once before timing
(one step5_index_summarize over every token, itself timed and reported as the
summary phase).

Layers: a model runs the step once per attention layer, each layer over its
own caches. The bench holds L copies of a workload's caches (summaries, KV,
k/z rings) at distinct addresses and step i runs on copy i mod L, with L
chosen so that the bytes the other L - 1 copies touch in between exceed three
times the 256 MB Infinity Cache: every step then reads its summaries and K/V
from HBM, not from a cache that still holds them from the step before. The
per-call times are taken the same way (back-to-back calls rotating over the
copies) and, for comparison, on one copy ("resident": the same buffers every
call, mostly served by the Infinity Cache).

Headline workload: decode16_ctx128k (16 decode rows, each with its own
131,072-token context, Student-t inputs) -> decode rows/s. Also reported
(see --extra): a 2,048-row chunked prefill at 32K (prefill tokens/s),
one decode row at a 1M-token context with a summary pass over a fresh
65,536-token span, and a plain device copy as the measured HBM ceiling. One
JSON line goes to stdout.
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
# HBM bytes per step5_sparse_attn call (attn_kernel + attn_mh_merge_kernel) on
# decode16_ctx128k, from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE;
# profiles/sparse_attn_hbm_counters_decode16_ctx128k.md), each scaled by what
# the counter reads for a 1 GiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).
# Valid only for the attention source the counters were taken on.
ATTN_TRAFFIC = {"source_sha256": "8e005b4a8c294e774eb30f8fdc448595d2531ce6d2ac4ff6e0bcd9e93a535eb1",
                "bytes_per_launch": 136713216}
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
METRIC = "sparse-attn decode rows/s at 128K ctx; indexer HBM GB/s as % of peak"
HEADLINE = "decode16_ctx128k"
RING_SLOTS = 520  # indexer k/z ring per sequence: one 512-token prompt chunk plus a region


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle's sample until this much time has passed")
    ap.add_argument("--extra", default="prefill2048_ctx32k,decode1_ctx1m,attn_geometry,qkv_projection,hbm_copy",
                    help="comma-separated extra lines to measure after the headline "
                         "(workload names, attn_geometry and/or hbm_copy; 'none' for none)")
    ap.add_argument("--eager", action="store_true", help="launch the calls directly, no HIP graphs")
    ap.add_argument("--steps-per-graph", type=int, default=0,
                    help="consecutive steps (one per layer copy) captured in one HIP graph; "
                         "0: one step per layer copy (a decode pass over the layers)")
    ap.add_argument("--no-resident", action="store_true",
                    help="skip the per-call times on one layer copy (so that a profiled run holds "
                         "only launches that rotate over the copies)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """Times a step made of several calls, over L layer copies, on the stream
    the calls run on.

    layers: one list of (name, fn) per layer copy, the same names in the same
    order. step(steps, per_graph): steps in turn on layer copy i mod L, with
    per_graph consecutive steps (one per layer copy: a decode pass over the
    model's layers) captured in ONE HIP graph and replayed (unless eager),
    a HIP event before every replay; steps not filling a graph run in a
    shorter one. per_call(rotate): each call captured `reps` times back to
    back in one graph, call k on layer k mod L (rotate) or on layer 0 every
    time (resident), replayed a few times; per-call time = event-timed replay
    / reps (what the call's kernels take, without the launch gap of a graph
    replay)."""

    def __init__(self, torch, layers, warmup, eager):
        self.torch = torch
        self.layers = layers
        self.names = [n for n, _ in layers[0]]
        self.eager = eager
        self.stream = torch.cuda.current_stream()
        self.graphs = {}
        for i in range(max(warmup, len(layers))):
            for _, f in layers[i % len(layers)]:
                f()
        torch.cuda.synchronize()

    def _capture(self, fns):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for f in fns:
                f()
        return g

    def _runner(self, first, count):
        """One run of `count` consecutive steps from layer copy `first`."""
        L = len(self.layers)
        fns = [f for i in range(count) for _, f in self.layers[(first + i) % L]]
        if self.eager:
            return lambda: [f() for f in fns]
        key = (first % L, count)
        if key not in self.graphs:
            self.graphs[key] = self._capture(fns)
        return self.graphs[key].replay

    def step(self, steps, per_graph, warmup=2):
        torch = self.torch
        L = len(self.layers)
        runs = []
        i = 0
        while i < steps:
            n = min(per_graph, steps - i)
            runs.append((self._runner(i, n), n))
            i += n
        for _ in range(warmup):
            for run, _ in runs:
                run()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(runs) + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j, (run, _) in enumerate(runs):
            evs[j].record(self.stream)
            run()
        evs[len(runs)].record(self.stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        gpu_ms = sum(evs[j].elapsed_time(evs[j + 1]) for j in range(len(runs)))
        return elapsed, gpu_ms / steps

    def per_call(self, rotate, reps=None, rounds=5):
        torch = self.torch
        L = len(self.layers)
        if reps is None:
            reps = L * max(1, -(-20 // L)) if rotate else 20
        out = {}
        for ci, name in enumerate(self.names):
            fns = [self.layers[(k % L) if rotate else 0][ci][1] for k in range(reps)]
            if self.eager:
                run = lambda fns=fns: [f() for f in fns]
            else:
                g = self._capture(fns)
                run = g.replay
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for _ in range(rounds):
                run()
            e1.record(self.stream)
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) * 1000.0 / (rounds * reps)
            del run
        return out


def event_time_us(torch, fn, reps, warm_s=0.0):
    """Average µs of fn over reps back-to-back calls, after one untimed call
    (or, with warm_s, untimed calls for about that many seconds, so that a
    long kernel is timed at the clocks a busy GPU holds)."""
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / reps


def workspaces(torch, s5, rows, R_cap, dev):
    ws1 = torch.empty(s5.step5_index_score_topk_workspace(rows, R_cap) + 256, dtype=torch.uint8,
                      device=dev)
    ws2 = torch.zeros(max(1, s5.step5_sparse_attn_workspace(rows)) + 256, dtype=torch.uint8,
                      device=dev)
    return ws1[(-ws1.data_ptr()) % 256:], ws2[(-ws2.data_ptr()) % 256:]


def attn_tokens(p):
    """Tokens one (row, KV head) attends at position p: 8 per selected region
    (min(512, p // 8) regions) plus the own region's p % 8 + 1."""
    return 8 * min(512, p // 8) + p % 8 + 1


def attn_bytes(rows_pos):
    """Algorithmic K+V bytes of one sparse-attention launch: per (row, KV head),
    the tokens it attends, 256 bytes each for K and for V."""
    return sum(4 * attn_tokens(p) * 256 * 2 for p in rows_pos)


def attn_flops(rows_pos):
    """Algorithmic flops of one sparse-attention launch: per (row, query
    head) and attended token, 128 multiply-adds for q.k and 128 for p.v."""
    return sum(16 * attn_tokens(p) * 128 * 4 for p in rows_pos)


# Bytes the other layer copies touch between two uses of one copy: at least
# three times the 256 MB Infinity Cache.
LAYER_REUSE_BYTES = 768 * 2 ** 20
MAX_LAYER_BYTES = 64 * 2 ** 30  # cap on the copies' memory (HBM holds 288 GB)


def layer_count(step_bytes, copy_bytes):
    """Layer copies for a step touching step_bytes, each copy holding
    copy_bytes: 1 + ceil(LAYER_REUSE_BYTES / step_bytes), within the cap."""
    want = 1 + -(-LAYER_REUSE_BYTES // max(1, step_bytes))
    cap = max(2, MAX_LAYER_BYTES // max(1, copy_bytes))
    return int(max(2, min(want, cap)))


def run_workload(name, args, torch, s5, W):
    """Builds the inputs, the summaries before the step and the layer copies,
    and times the step. Returns (result dict, inputs dict, summaries)."""
    wl = W.WORKLOADS[name]
    dev = "cuda"
    log(f"{name}: generating inputs")
    d = W.make_case(wl, args.seed, dev)
    rows, T, B = d["rows"], d["cache_tokens"], d["batch"]
    R_cap = T // 8
    eps = W.NORM_EPS
    scale = 1.0 / math.sqrt(W.HEAD_DIM)
    pos = [int(x) for x in d["row_pos"].cpu()]
    res = {"workload": name, "rows": rows, "context_tokens": T, "sequences": B,
           "row_positions": sorted(set(pos)) if len(set(pos)) <= 4 else [min(pos), max(pos)],
           "candidates_per_row": sorted({p // 8 for p in pos}) if len(set(pos)) <= 4
           else [min(pos) // 8, max(pos) // 8]}

    # ---- summaries before the step (and the summary-phase measurement)
    if wl.tie_heavy:
        S = d["summary"]
        S_fresh = torch.zeros((1, wl.fresh_tokens // 8, 4, 64), dtype=torch.uint8, device=dev)
        full_pass = lambda: s5.step5_index_summarize(d["fresh_k"], d["fresh_z"], 0, d["ln_w"],
                                                     d["ln_b"], eps, d["rope"], S_fresh)
        pass_tokens = wl.fresh_tokens
        pass_name = f"fresh span of {wl.fresh_tokens} tokens"
    else:
        S = torch.zeros((B, R_cap, 4, 64), dtype=torch.uint8, device=dev)
        prefix = T - wl.prefill_chunk if wl.prefill_chunk else T
        kp, zp = d["k_idx"][:, :prefix], d["z_idx"][:, :prefix]
        full_pass = lambda: s5.step5_index_summarize(kp, zp, 0, d["ln_w"], d["ln_b"], eps,
                                                     d["rope"], S)
        pass_tokens = B * prefix
        pass_name = f"{B} x {prefix} tokens"
    log(f"{name}: summary pass over {pass_name}")
    summ_us = event_time_us(torch, full_pass, 10, warm_s=0.5)
    summ_bytes = pass_tokens * 1024 + (pass_tokens // 8) * 256
    res["summary_pass"] = {"span": pass_name, "us": round(summ_us, 1),
                           "GBs": round(summ_bytes / summ_us / 1e3, 1),
                           "frac_hbm": round(summ_bytes / summ_us / 1e3 / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes": summ_bytes}

    # ---- layer copies of the caches the step reads and writes
    a_bytes = attn_bytes(pos)
    sc_bytes = sum(p // 8 for p in pos) * 256
    copy_bytes = (d["k_cache"].numel() * 2 * 2 + S.numel())
    # bytes a step touches: what the rows gather, but no more than the caches
    # hold (a prompt chunk's rows re-read one sequence's K/V many times)
    step_bytes = min(a_bytes + sc_bytes, copy_bytes)
    L = layer_count(step_bytes, copy_bytes)
    log(f"{name}: {L} layer copies ({copy_bytes * L / 2 ** 30:.1f} GiB)")
    ring = None
    if not wl.prefill_chunk and not wl.tie_heavy:
        ring = ring_before_step(torch, d, RING_SLOTS)
    layers = []
    for li in range(L):
        first = li == 0
        lay = {"S": S if first else S.clone(),
               "k_cache": d["k_cache"] if first else d["k_cache"].clone(),
               "v_cache": d["v_cache"] if first else d["v_cache"].clone()}
        if ring is not None:
            lay["k_ring"] = ring[0] if first else ring[0].clone()
            lay["z_ring"] = ring[1] if first else ring[1].clone()
        layers.append(lay)

    # ---- the step, per layer copy
    ids = torch.empty((rows, 4, 512), dtype=torch.int32, device=dev)
    out = torch.empty((rows, 16, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=dev)
    ws1, ws2 = workspaces(torch, s5, rows, R_cap, dev)
    one_per_seq = len(set(d["row_seq"].tolist())) == rows
    fused_select = ring is not None and one_per_seq  # the append runs inside the selection's call
    summ_step_tokens = wl.prefill_chunk
    if ring is not None:
        rs, rp = d["row_seq"].long(), d["row_pos"]
        k_new, z_new = d["k_idx"][rs, rp].contiguous(), d["z_idx"][rs, rp].contiguous()

    def layer_calls(lay):
        calls = []
        Sl = lay["S"]
        if wl.prefill_chunk:
            t0 = T - wl.prefill_chunk
            kc_, zc_ = d["k_idx"][:, t0:], d["z_idx"][:, t0:]
            calls.append(("summarize", lambda: s5.step5_index_summarize(
                kc_, zc_, t0, d["ln_w"], d["ln_b"], eps, d["rope"], Sl)))
        elif ring is not None:
            # the rings hold the open regions' earlier tokens; each step appends
            # the rows' own tokens (the last of their regions here)
            if one_per_seq:
                # rows of distinct sequences: the append runs inside the
                # selection's launch (step5_index_append_score_topk)
                calls.append(("append_score_topk", lambda: s5.step5_index_append_score_topk(
                    k_new, z_new, lay["k_ring"], lay["z_ring"], d["ln_w"], d["ln_b"], eps,
                    d["q_idx"], d["w_head"], d["row_seq"], d["row_pos"], Sl, ids, rope=d["rope"],
                    q_norm_w=d["q_norm_w"], q_eps=eps, workspace=ws1)))
            else:
                calls.append(("append", lambda: s5.step5_index_append(
                    k_new, z_new, d["row_seq"], d["row_pos"], lay["k_ring"], lay["z_ring"],
                    d["ln_w"], d["ln_b"], eps, d["rope"], Sl, one_per_seq=False)))
        if wl.tie_heavy:
            calls.append(("score_topk", lambda: s5.step5_index_score_topk(
                d["q8"], d["w_head"], d["row_seq"], d["row_pos"], Sl, ids, q_is_e4m3=True,
                workspace=ws1)))
        elif not fused_select:
            calls.append(("score_topk", lambda: s5.step5_index_score_topk(
                d["q_idx"], d["w_head"], d["row_seq"], d["row_pos"], Sl, ids,
                q_norm_w=d["q_norm_w"], q_eps=eps, rope=d["rope"], workspace=ws1)))
        calls.append(("sparse_attn", lambda: s5.step5_sparse_attn(
            d["q"], lay["k_cache"], lay["v_cache"], ids, d["row_seq"], d["row_pos"], scale, out,
            lse, workspace=ws2)))
        return calls

    steps = args.steps if name == HEADLINE else max(5, min(args.steps, 20))
    per_graph = L if args.steps_per_graph == 0 else args.steps_per_graph
    log(f"{name}: timing {steps} steps over {L} layer copies, {per_graph} steps per graph")
    timer = Timer(torch, [layer_calls(lay) for lay in layers], args.warmup, args.eager)
    elapsed, gpu_step_ms = timer.step(steps, per_graph)
    one_per_graph = None
    if per_graph != 1 and not args.eager:
        e1, g1 = timer.step(steps, 1)
        one_per_graph = {"ms_per_step": round(e1 * 1000.0 / steps, 4),
                         "gpu_ms_per_step": round(g1, 4),
                         "rows_per_s": round(rows * steps / e1, 1)}
    log(f"{name}: per-call times (rotating, then resident)")
    per_call = timer.per_call(rotate=True)
    per_res = {} if args.no_resident else timer.per_call(rotate=False)
    del timer
    ms_per_step = elapsed * 1000.0 / steps

    # the selection's call (with the appends inside it when fused)
    sel_name = "append_score_topk" if fused_select else "score_topk"
    sc_flops = sum(p // 8 for p in pos) * 16 * 64 * 2
    a_flops = attn_flops(pos)
    res.update({
        "layers": L,
        "layer_reuse_bytes": (L - 1) * step_bytes,
        "steps_per_graph": per_graph,
        "one_step_per_graph": one_per_graph,
        "steps": steps,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_step_ms, 4),
        "rows_per_s": round(rows * steps / elapsed, 1),
        "call_us": {k: round(v, 2) for k, v in per_call.items()},
        "call_us_resident": {k: round(v, 2) for k, v in per_res.items()},
    })

    def rate(nbytes, us):
        return {"GBs": round(nbytes / us / 1e3, 1),
                "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}

    def mfma(flops, us, peaks):
        r = {"TFLOPs": round(flops / us / 1e6, 2)}
        for k, p in peaks:
            r[k] = round(flops / us / 1e6 / p, 5)
        return r

    if wl.prefill_chunk:
        # A prompt chunk's rows share one sequence: the attention and the
        # scoring re-read the same 64 MiB of K/V and 1 MiB of summaries many
        # times over (through L2 and the Infinity Cache). Their bound is the
        # matrix cores, so they are reported against the MFMA peaks; the
        # logical bytes (what per-row gathers would move) are context only.
        res["sparse_attn"] = {"algorithmic_flops": a_flops, "logical_bytes": a_bytes,
                              **mfma(a_flops, per_call["sparse_attn"],
                                     [("frac_bf16_mfma", BF16_PEAK_TFLOPS)]),
                              "logical_GBs": round(a_bytes / per_call["sparse_attn"] / 1e3, 1)}
        res["score_topk"] = {"algorithmic_flops": sc_flops, "logical_summary_bytes": sc_bytes,
                             **mfma(sc_flops, per_call[sel_name],
                                    [("frac_fp8_mfma", FP8_PEAK_TFLOPS),
                                     ("frac_bf16_mfma", BF16_PEAK_TFLOPS)]),
                             "logical_GBs": round(sc_bytes / per_call[sel_name] / 1e3, 1)}
    else:
        res["sparse_attn"] = {"algorithmic_bytes": a_bytes, **rate(a_bytes, per_call["sparse_attn"])}
        if per_res:
            res["sparse_attn"]["resident"] = rate(a_bytes, per_res["sparse_attn"])
        sel = {"summary_bytes": sc_bytes, "score_flops": sc_flops,
               **rate(sc_bytes, per_call[sel_name]),
               **mfma(sc_flops, per_call[sel_name], [("frac_fp8_mfma", FP8_PEAK_TFLOPS),
                                                     ("frac_bf16_mfma", BF16_PEAK_TFLOPS)])}
        if per_res:
            sel["resident"] = rate(sc_bytes, per_res[sel_name])
        if fused_select:
            # the call also runs the rows' appends: per row its token's k and z
            # read and written to the ring (2 KB); per completed region its 8
            # tokens' k and z (8 KB) read and 256 B written
            done = sum(1 for p in pos if p % 8 == 7)
            sel["append_bytes"] = rows * 2048 + done * (8 * 1024 + 256)
            sel["ring_slots"] = RING_SLOTS
        res[sel_name] = sel
    if "summarize" in per_call:
        b = summ_step_tokens * 1024 + (summ_step_tokens // 8) * 256
        res["summarize_in_step"] = {"tokens": summ_step_tokens, "algorithmic_bytes": b,
                                    "GBs": round(b / per_call["summarize"] / 1e3, 1)}
    if "append" in per_call:
        done = sum(1 for p in pos if p % 8 == 7)
        b = rows * 2048 + done * (8 * 1024 + 256)
        res["append_in_step"] = {"rows": rows, "regions_completed": done, "algorithmic_bytes": b,
                                 "ring_slots": RING_SLOTS,
                                 "GBs": round(b / per_call["append"] / 1e3, 1)}
    if wl.prefill_chunk:
        res["prefill_tokens_per_s"] = round(wl.prefill_chunk * steps / elapsed, 1)
    del layers
    return res, d, S


def ring_before_step(torch, d, slots):
    """k/z rings [B, slots, 4, 64] holding, for every row, the tokens of its
    own region before the row's position (what earlier appends left there)."""
    k, z = d["k_idx"], d["z_idx"]
    k_ring = torch.zeros((k.shape[0], slots) + tuple(k.shape[2:]), dtype=k.dtype, device=k.device)
    z_ring = torch.zeros_like(k_ring)
    for s, p in zip(d["row_seq"].tolist(), d["row_pos"].tolist()):
        for t in range(p - p % 8, p):
            k_ring[s, t % slots] = k[s, t]
            z_ring[s, t % slots] = z[s, t]
    return k_ring, z_ring


def attn_traffic(workload):
    """Measured HBM bytes per attention call, or None when the workload or the
    attention source differs from the one the counters were taken on."""
    import hashlib
    if workload != HEADLINE:
        return None
    return ATTN_TRAFFIC["bytes_per_launch"] if attn_source_sha() == ATTN_TRAFFIC["source_sha256"] else None


def attn_source_sha():
    """sha256 over the sources of the decode attention call: attn_kernel and
    the tile predicate it evaluates (attn.hip, attn_tile.hpp) and the split
    merge (attn_mh.hip)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("attn.hip", "attn_tile.hpp", "attn_mh.hip"):
        with open(os.path.join(ROOT, "long_context_sparse_indexer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def attn_geometry(torch, s5):
    """step5_sparse_attn alone at the 128K decode shape (16 rows, each its own
    131,072-token sequence at position 131,071, 512 random regions per (row,
    KV head)) for 4, 8 and 16 query heads per KV head of 128 dims and 16 of
    192 (Step-5's own layer shape). Back-to-back calls rotate over 6 random
    selections, so a call finds little of its K/V in the Infinity Cache.
    Algorithmic bytes: the K and V rows the selection names, D x 2 bytes
    each, per (row, KV head)."""
    rows, T, NSEL = 16, 131072, 6
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    pos = torch.full((rows,), T - 1, dtype=torch.int64, device=dev)
    seq = torch.arange(rows, dtype=torch.int32, device=dev)
    sels = [torch.stack([torch.randperm(T // 8 - 1, generator=g, device=dev)[:512]
                         for _ in range(rows * 4)]).to(torch.int32).view(rows, 4, 512).contiguous()
            for _ in range(NSEL)]
    res = {"shape": f"{rows} rows x {T} tokens, 512 regions + own per (row, KV head)",
           "selections_rotated": NSEL}
    for D, hqs in ((128, (16, 32, 64)), (192, (64,))):
        k = torch.randn((rows, T, 4, D), generator=g, device=dev, dtype=torch.bfloat16)
        v = torch.randn((rows, T, 4, D), generator=g, device=dev, dtype=torch.bfloat16)
        for Hq in hqs:
            q = torch.randn((rows, Hq, D), generator=g, device=dev, dtype=torch.bfloat16)
            out = torch.empty((rows, Hq, D), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((rows, Hq), dtype=torch.float32, device=dev)
            nb = s5.step5_sparse_attn_workspace(rows, Hq, D)
            ws = torch.zeros(max(1, nb) + 256, dtype=torch.uint8, device=dev)
            ws = ws[(-ws.data_ptr()) % 256:]
            layers = [[("attn", (lambda ids=ids: s5.step5_sparse_attn(
                q, k, v, ids, seq, pos, 1.0 / math.sqrt(D), out, lse, workspace=ws)))]
                for ids in sels]
            us = Timer(torch, layers, 3, False).per_call(rotate=True)["attn"]
            b = rows * 4 * (8 * 512 + 8) * D * 2 * 2
            res[f"q{Hq}_d{D}"] = {"heads_per_kv": Hq // 4, "us": round(us, 2),
                                  "algorithmic_bytes": b, "GBs": round(b / us / 1e3, 1),
                                  "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
        del k, v
    return res


def qkv_projection(torch, s5):
    """step5_qkv_index_project at the layer's shape (hidden 4,096; q 16 x 128,
    k and v 4 x 128, indexer q 16 x 64, k and z 4 x 64, a 16-column gate:
    4,624 columns) for the decode shape (16 rows) and a prompt chunk (2,048
    rows), with synthetic bf16 weights. Back-to-back calls rotate over layer
    copies of the weight (a model's layers each have their own), enough that
    the weight is read from HBM. Algorithmic work: 2 x rows x 4,624 x 4,096
    flop; bytes: the weight (37.9 MB) plus the hidden rows and outputs."""
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(91)
    widths = s5.proj_widths()
    N, H = sum(widths), 4096
    w0 = (torch.randn((N, H), generator=g, device=dev) / 64).to(torch.bfloat16)
    L = layer_count(N * H * 2, N * H * 2)
    ws = [w0] + [w0.clone() for _ in range(L - 1)]
    res = {"shape": f"hidden {H} -> {N} columns (q, k, v, index_q, index_k, index_z, gate)",
           "weight_copies_rotated": L}
    for rows in (16, 2048):
        h = torch.randn((rows, H), generator=g, device=dev).to(torch.bfloat16)
        outs = [torch.empty((rows, wd), dtype=torch.bfloat16, device=dev) for wd in widths]
        layers = [[("proj", (lambda w=w: s5.step5_qkv_index_project(h, w, outs)))] for w in ws]
        us = Timer(torch, layers, 3, False).per_call(rotate=True)["proj"]
        flop = 2.0 * rows * N * H
        byts = N * H * 2 + rows * H * 2 + rows * N * 2
        res[f"rows{rows}"] = {"us": round(us, 2), "TFLOPs": round(flop / us / 1e6, 1),
                              "frac_bf16_mfma": round(flop / us / 1e6 / BF16_PEAK_TFLOPS, 4),
                              "GBs": round(byts / us / 1e3, 1),
                              "frac_hbm": round(byts / us / 1e3 / HBM_PEAK_GBS, 4)}
        del h, outs
    del ws, w0
    return res


def copy_ceiling(torch):
    """A plain device-to-device copy of 1 GiB: the HBM rate a streaming kernel
    reaches on this GPU (read + write bytes per second)."""
    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    us = event_time_us(torch, lambda: y.copy_(x), 10)
    gbs = 2 * 4 * n / us / 1e3
    del x, y
    return {"bytes_per_copy": 2 * 4 * n, "us": round(us, 1), "GBs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no sharding or collectives are built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_indexer_amd as s5
    import workloads as W

    torch.cuda.init()
    head, d, S = run_workload(args.workload, args, torch, s5, W)
    wl = W.WORKLOADS[args.workload]
    cpu = None
    if not args.no_cpu_baseline:
        log("oracle baseline on the host")
        cpu = cpu_baseline(d, wl, args.cpu_rows, args.cpu_seconds, torch)
    del d, S
    torch.cuda.empty_cache()

    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != "none"]:
        if name == "hbm_copy":
            log("plain copy of 1 GiB")
            extra[name] = copy_ceiling(torch)
        elif name == "qkv_projection":
            log("fused qkv + indexer projection at the layer's shape")
            extra[name] = qkv_projection(torch, s5)
            torch.cuda.empty_cache()
        elif name == "attn_geometry":
            log("sparse attention of other query-head geometries at the 128K decode shape")
            extra[name] = attn_geometry(torch, s5)
            torch.cuda.empty_cache()
        elif name != args.workload:
            r, dd, SS = run_workload(name, args, torch, s5, W)
            del dd, SS
            torch.cuda.empty_cache()
            extra[name] = r

    sa = head["sparse_attn"]
    result = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": head["rows"], "context_tokens": head["context_tokens"],
                   "sequences": head["sequences"], "row_position": head["row_positions"][0],
                   "candidates_per_row": head["candidates_per_row"][0], "topk": 512, "region": 8,
                   "idx_heads": 16, "kv_groups": 4, "q_heads": 16, "head_dim": 128,
                   "inputs": wl.dist, "layer_copies": head["layers"]},
        "roofline": ({"bound": "hbm",
                      "kernel": "step5_sparse_attn (attn_kernel, split states merged in the launch)",
                      "achieved": sa["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": sa["frac_hbm"], "traffic": attn_traffic(args.workload),
                      "algorithmic_bytes_per_launch": sa["algorithmic_bytes"],
                      "layer_copies": head["layers"]} if "GBs" in sa else
                     {"bound": "mfma",
                      "kernel": "step5_sparse_attn (attn_tile_kernel, the context sweep)",
                      "achieved": sa["TFLOPs"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": sa["frac_bf16_mfma"], "traffic": None,
                      "algorithmic_flops_per_launch": sa["algorithmic_flops"],
                      "layer_copies": head["layers"]}),
        "phases": {"graph_replay": not args.eager, **{k: v for k, v in head.items()
                                                      if k not in ("workload",)}},
    }
    if extra:
        result["extra"] = extra
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def host_info():
    """The host CPU's model name and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": avail, "os_cpu_count": os.cpu_count()}


def cpu_baseline(d, wl, nrows, seconds, torch):
    """The oracle (unchanged) on a bounded sample of the same decode step,
    twice: on every CPU this process may use (the first `nrows` rows, each
    over its own sequence) and on one core (the first row), each repeated
    until `seconds` have passed. The oracle builds its own summaries of those
    sequences first (untimed, like the GPU's cache); the timed part is the
    step: the rows' tokens appended (ring + the region each completes), q
    prep, scores, top-512 selection and attention."""
    import numpy as np
    from oracle import oracle as orc
    import workloads as W

    host = host_info()
    nth_all = int(os.environ.get("STEP5_ORACLE_THREADS") or os.environ.get("OMP_NUM_THREADS")
                  or host["nproc"])
    rows_all = list(range(min(nrows, d["rows"])))
    seqs = sorted({int(d["row_seq"][r]) for r in rows_all})
    smap = {s: i for i, s in enumerate(seqs)}
    T = d["cache_tokens"]
    rope = W.bits16(d["rope"])
    lnw, lnb = d["ln_w"].cpu().numpy(), d["ln_b"].cpu().numpy()
    qnw = None if wl.tie_heavy else d["q_norm_w"].cpu().numpy()
    if wl.tie_heavy:
        Sh = W.bits8(d["summary"][seqs])
        q8all = W.bits8(d["q8"])
    else:
        k16 = np.concatenate([W.bits16(d["k_idx"][s:s + 1]) for s in seqs])
        z16 = np.concatenate([W.bits16(d["z_idx"][s:s + 1]) for s in seqs])
        Sh = orc.summarize(k16, z16, 0, lnw, lnb, W.NORM_EPS, rope, nthreads=nth_all)
        qidx = W.bits16(d["q_idx"])
    kc = np.concatenate([W.bits16(d["k_cache"][s:s + 1]) for s in seqs])
    vc = np.concatenate([W.bits16(d["v_cache"][s:s + 1]) for s in seqs])
    w = d["w_head"].cpu().numpy()
    qall = W.bits16(d["q"])
    pos_all = d["row_pos"].cpu().numpy()

    def leg(rows, nth):
        pos = pos_all[rows]
        seq = np.array([smap[int(d["row_seq"][r])] for r in rows], np.int32)
        q = qall[rows]
        if not wl.tie_heavy:
            # the rings as the GPU step starts them, the rows' new tokens
            k_ring = np.zeros((len(seqs), RING_SLOTS, 4, 64), np.uint16)
            z_ring = np.zeros_like(k_ring)
            for i, r in enumerate(rows):
                s, p = smap[int(d["row_seq"][r])], int(pos[i])
                for t in range(p - p % 8, p):
                    k_ring[s, t % RING_SLOTS] = k16[s, t]
                    z_ring[s, t % RING_SLOTS] = z16[s, t]
            k_new = np.stack([k16[seq[i], pos[i]] for i in range(len(rows))])
            z_new = np.stack([z16[seq[i], pos[i]] for i in range(len(rows))])

        def one_step():
            if not wl.tie_heavy:
                orc.append(k_new, z_new, seq, pos, k_ring, z_ring, lnw, lnb, W.NORM_EPS, rope,
                           Sh)
                q8 = orc.q_prep(qidx[rows], qnw, W.NORM_EPS, rope, pos, nthreads=nth)
            else:
                q8 = q8all[rows]
            sc = orc.score(q8, w, seq, pos, Sh, nthreads=nth)
            ids, _ = orc.select(sc, pos, 512, nthreads=nth)
            orc.attend(q, kc, vc, ids, seq, pos, 1.0 / math.sqrt(W.HEAD_DIM), nthreads=nth)

        reps = 0
        t0 = time.perf_counter()
        while True:
            one_step()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
        return round(len(rows) * reps / dt, 3), reps, dt

    v_all, reps_all, dt_all = leg(rows_all, nth_all)
    v_one, reps_one, dt_one = leg(rows_all[:1], 1)
    what = ("cache append (ring + own-region summary), q prep, scores, top-512, attention"
            if not wl.tie_heavy else "scores, top-512, attention (q given as e4m3)")
    return {"value": v_all, "unit": "rows/s", "cores": nth_all, "kind": "oracle",
            "sample": f"rows 0..{len(rows_all) - 1} of {wl.name} ({len(rows_all)} of {d['rows']} "
                      f"rows, each its own {T}-token sequence): {what}; repeated {reps_all} "
                      f"times in {dt_all:.1f} s on {nth_all} threads",
            "single_core": {"value": v_one, "unit": "rows/s", "cores": 1,
                            "sample": f"row 0 of {wl.name}, the same step, repeated {reps_one} "
                                      f"times in {dt_one:.1f} s on 1 thread"},
            "host": host}


if __name__ == "__main__":
    main()
