"""The three calls captured in HIP graphs (as bench.py replays them): every
replay, with eager work and synchronisations between replays, matches the
eager result bit for bit. The kernels clear nothing with memset nodes, so
nothing in a replay depends on state a previous replay left."""
import math

import pytest
import torch

import workloads as W
import parity as P
import long_context_sparse_indexer_amd as s5

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode1_ctx6000", "decode16_ctx128k"])
def test_graph_replays_match_eager(name):
    dev = "cuda"
    kw = {} if name == "decode1_ctx6000" else {"cache_tokens": 16384}
    d = W.make_case(W.WORKLOADS[name], 31, dev, **kw)
    P.say(f"[case] graph {name}")
    rows, T, B = d["rows"], d["cache_tokens"], d["batch"]
    R_cap = T // 8
    S = torch.zeros((B, R_cap, 4, 64), dtype=torch.uint8, device=dev)
    s5.step5_index_summarize(d["k_idx"], d["z_idx"], 0, d["ln_w"], d["ln_b"], P.EPS, d["rope"], S)
    ws1 = torch.empty(s5.step5_index_score_topk_workspace(rows, R_cap), dtype=torch.uint8, device=dev)
    ws2 = torch.zeros(max(1, s5.step5_sparse_attn_workspace(rows)), dtype=torch.uint8, device=dev)
    own0 = (T - 1) // 8 * 8
    ids = torch.empty((rows, 4, 512), dtype=torch.int32, device=dev)
    sc = torch.empty((rows, 4, 512), dtype=torch.float32, device=dev)
    out = torch.empty((rows, 16, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, 16), dtype=torch.float32, device=dev)

    def step():
        s5.step5_index_summarize(d["k_idx"][:, own0:own0 + 8], d["z_idx"][:, own0:own0 + 8], own0,
                                 d["ln_w"], d["ln_b"], P.EPS, d["rope"], S)
        s5.step5_index_score_topk(d["q_idx"], d["w_head"], d["row_seq"], d["row_pos"], S, ids, sc,
                                  q_norm_w=d["q_norm_w"], q_eps=P.EPS, rope=d["rope"], workspace=ws1)
        s5.step5_sparse_attn(d["q"], d["k_cache"], d["v_cache"], ids, d["row_seq"], d["row_pos"],
                             1 / math.sqrt(128), out, lse, workspace=ws2)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (S, ids, sc, out, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (ids, sc, lse):
            t.fill_(-3)
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((S, ids, sc, out, lse), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (name, rep)
        step()                                   # eager work between replays
        torch.cuda.synchronize()
