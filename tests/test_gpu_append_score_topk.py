"""GPU parity of step5_index_append_score_topk: a decode step's cache append
and selection in one call give, bit for bit, what step5_index_append (one row
per sequence) followed by step5_index_score_topk give: the same ids and
scores, the same rings and the same summaries; and a stream of such calls
leaves the summaries the oracle's batch summary writes.

Source: TensorFold pull request #903 "Step-5-Preview on one 256 GB Mac"
(indexer commit note: every completed region summarised, q prep, scores, top
512; prompt-path commit note: the indexer's k and z in rings).
"""
import numpy as np
import pytest
import torch

import workloads as W
import parity as P
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _state(B, slots, R_cap, seed):
    g = torch.Generator().manual_seed(seed)
    k_ring = torch.randn(B, slots, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    z_ring = torch.randn(B, slots, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    S = torch.randint(0, 255, (B, R_cap, 4, 64), generator=g, dtype=torch.uint8)
    S[(S & 0x7F) == 0x7F] = 0   # no NaN codes
    return k_ring, z_ring, S.to(DEV)


def _both(d, k_new, z_new, q, seq, pos, k_ring, z_ring, S):
    """The fused call on one copy of the state, the two calls on another."""
    rows = q.shape[0]
    out = []
    for fused in (True, False):
        kr, zr, Sx = k_ring.clone(), z_ring.clone(), S.clone()
        ids = torch.full((rows, 4, 512), -7, dtype=torch.int32, device=DEV)
        sc = torch.full((rows, 4, 512), -7.0, dtype=torch.float32, device=DEV)
        common = dict(q_norm_w=d["q_norm_w"], q_eps=P.EPS, rope=d["rope"])
        if fused:
            P.s5.step5_index_append_score_topk(k_new, z_new, kr, zr, d["ln_w"], d["ln_b"], P.EPS,
                                               q, d["w_head"], seq, pos, Sx, ids, sc, **common)
        else:
            P.s5.step5_index_append(k_new, z_new, seq, pos, kr, zr, d["ln_w"], d["ln_b"], P.EPS,
                                    d["rope"], Sx, one_per_seq=True)
            P.s5.step5_index_score_topk(q, d["w_head"], seq, pos, Sx, ids, sc, **common)
        torch.cuda.synchronize()
        out.append((ids, sc, kr, zr, Sx))
    return out


def _equal(a, b, where):
    names = ("ids", "scores", "k ring", "z ring", "summary")
    for n, x, y in zip(names, a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{where}: {n} differ"


@pytest.mark.parametrize("rows", [16, 72])
def test_fused_equals_two_calls(rows):
    """rows sequences (16: the exact scorer; 72: intervals and rescoring) of
    3,000 tokens; positions mixed so some tokens complete their region,
    others not, one row past the rope table and one of no sequence."""
    T, slots = 3000, 24
    d = W.make_case(W.WORKLOADS["decode8_ctx3000"], 5 + rows, DEV, cache_tokens=T, rows=rows,
                    batch=rows, with_kv=False)
    R_cap = T // 8
    g = torch.Generator().manual_seed(rows)
    pos = torch.randint(8, T, (rows,), generator=g, dtype=torch.int64)
    pos[::3] = pos[::3] | 7               # these complete their region
    pos[1] = T + 5                        # past the rope table: skipped by both halves
    seq = torch.arange(rows, dtype=torch.int32)
    seq[2] = -1                           # no sequence
    pos, seq = pos.to(DEV), seq.to(DEV)
    k_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    z_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    k_ring, z_ring, S = _state(rows, slots, R_cap, rows)
    P.say(f"[case] append + score_topk fused vs two calls, {rows} rows")
    a, b = _both(d, k_new, z_new, d["q_idx"], seq, pos, k_ring, z_ring, S)
    _equal(a, b, f"rows={rows}")
    assert not torch.equal(a[4], S), "no region was summarised"


def test_fused_stream_equals_batch_summary():
    """3 sequences of 101 tokens, one token per call per sequence through
    the fused call (a 24-slot ring): every call's selection equals the two
    calls', and the summaries at the end equal the oracle's batch summary."""
    d = W.make_case(W.WORKLOADS["decode8_ctx3000"], 23, "cpu", cache_tokens=101, rows=3, batch=3,
                    with_kv=False)
    B, T, slots, R_cap = 3, 101, 24, 14
    k, z = d["k_idx"].to(DEV), d["z_idx"].to(DEV)
    dd = {n: d[n].to(DEV) for n in ("q_norm_w", "rope", "ln_w", "ln_b", "w_head")}
    k_ring = torch.zeros((B, slots, 4, 64), dtype=torch.bfloat16, device=DEV)
    z_ring = torch.zeros_like(k_ring)
    S = torch.full((B, R_cap, 4, 64), 0x55, dtype=torch.uint8, device=DEV)
    g = torch.Generator().manual_seed(3)
    seq = torch.arange(B, dtype=torch.int32, device=DEV)
    P.say("[case] fused append + score_topk stream, B=3 T=101")
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        q = torch.randn(B, 16, 64, generator=g).to(torch.bfloat16).to(DEV)
        a, b = _both(dd, k[:, t].contiguous(), z[:, t].contiguous(), q, seq, pos, k_ring, z_ring, S)
        _equal(a, b, f"t={t}")
        k_ring, z_ring, S = a[2], a[3], a[4]
    base = np.full((B, R_cap, 4, 64), 0x55, np.uint8)
    O = orc.summarize(P.host16(d["k_idx"]), P.host16(d["z_idx"]), 0, d["ln_w"].numpy(),
                      d["ln_b"].numpy(), P.EPS, P.host16(d["rope"]), R_cap=R_cap, summary=base)
    assert np.array_equal(S.cpu().numpy(), O)


def test_fused_multi_chunk_selection():
    """2 rows over 40,000 regions (320,000 tokens): the selection runs in 3
    chunks per unit plus a merge by the last chunk to finish, and the append
    workgroups sit beside every chunk column (only the first runs them)."""
    rows, R_cap, slots = 2, 40000, 16
    g = torch.Generator().manual_seed(77)
    T = R_cap * 8
    d = {"q_norm_w": (torch.randn(64, generator=g) * 0.1).to(DEV),
         "ln_w": (torch.randn(64, generator=g) * 0.1 + 1).to(DEV),
         "ln_b": (torch.randn(64, generator=g) * 0.1).to(DEV),
         "w_head": torch.rand(16, generator=g).to(DEV),
         "rope": torch.rand(T, 32, generator=g).to(torch.bfloat16).to(DEV)}
    pos = torch.tensor([T - 1, T - 9 - 3], dtype=torch.int64, device=DEV)   # completes / not
    seq = torch.arange(rows, dtype=torch.int32, device=DEV)
    q = torch.randn(rows, 16, 64, generator=g).to(torch.bfloat16).to(DEV)
    k_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    z_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    k_ring, z_ring, S = _state(rows, slots, R_cap, 78)
    P.say(f"[case] fused append + score_topk, {rows} rows x {R_cap} regions (chunked selection)")
    a, b = _both(d, k_new, z_new, q, seq, pos, k_ring, z_ring, S)
    _equal(a, b, "multi-chunk")
    assert not torch.equal(a[4], S)


@pytest.mark.parametrize("rows,R_cap", [(72, 2000), (72, 5000), (66, 20000)])
def test_fused_interval_selection_with_a_cut(rows, R_cap):
    """More than 64 rows, so the selection works on score intervals with exact
    rescoring, over more than 512 candidates per row so the threshold,
    compaction and rescoring all run beside the append workgroups: 2,000
    regions (intervals computed inside the selection), 5,000 (intervals
    stored by the score pass, one chunk per unit) and 20,000 (stored
    intervals, two chunks per unit and a merge)."""
    slots = 16
    g = torch.Generator().manual_seed(rows + R_cap)
    T = R_cap * 8
    d = {"q_norm_w": (torch.randn(64, generator=g) * 0.1).to(DEV),
         "ln_w": (torch.randn(64, generator=g) * 0.1 + 1).to(DEV),
         "ln_b": (torch.randn(64, generator=g) * 0.1).to(DEV),
         "w_head": torch.rand(16, generator=g).to(DEV),
         "rope": torch.rand(T, 32, generator=g).to(torch.bfloat16).to(DEV)}
    pos = T - 1 - torch.randint(0, 8 * 300, (rows,), generator=g, dtype=torch.int64)
    pos[::4] = pos[::4] | 7                 # these complete their region
    seq = torch.randperm(rows, generator=g).to(torch.int32)
    pos, seq = pos.to(DEV), seq.to(DEV)
    q = torch.randn(rows, 16, 64, generator=g).to(torch.bfloat16).to(DEV)
    k_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    z_new = torch.randn(rows, 4, 64, generator=g).to(torch.bfloat16).to(DEV)
    k_ring, z_ring, S = _state(rows, slots, R_cap, rows * 7 + 1)
    P.say(f"[case] fused append + score_topk (intervals), {rows} rows x {R_cap} regions")
    a, b = _both(d, k_new, z_new, q, seq, pos, k_ring, z_ring, S)
    _equal(a, b, f"rows={rows} R_cap={R_cap}")
    assert not torch.equal(a[4], S)
    assert bool((a[0][:, :, 511] >= 0).all()), "every unit selects 512"
