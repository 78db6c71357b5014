"""GPU parity at the full 128K decode shape, every row: 16 sequences of
131,072 tokens (Student-t inputs), one decode row each at position 131,071.

The step is run the way the benchmark times it: the summaries of the first
131,064 tokens of every sequence by step5_index_summarize, then
step5_index_append_score_topk, which appends each row's token (its region's
7 earlier tokens already in the k/z ring) and so completes region 16,383,
and selects the rows' top 512 per KV group; then step5_sparse_attn over the
picks. Against the oracle on the same bytes:

  * all 16 x 16,384 x 4 x 64 summary codes, bit-exact (the region the append
    completes included);
  * all 16 x 4 selections (ids and scores, position by position), strict: no
    near-tie excusal;
  * the plain step5_index_score_topk on the same summaries gives the same ids
    and scores as the fused call;
  * attention of all 16 rows within 2e-3 + 1e-2 |ref| of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as s5
import parity as P
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
SLOTS = 520


@pytest.fixture(scope="module")
def case():
    d = W.make_case(W.WORKLOADS["decode16_ctx128k"], 41, DEV)
    P.say("[case] decode16_ctx128k seed=41, all 16 rows")
    rows, T = d["rows"], d["cache_tokens"]
    assert rows == 16 and T == 131072 and all(int(p) == T - 1 for p in d["row_pos"].cpu())
    # summaries of the regions before the rows' own, then the fused decode call
    S = torch.full((16, T // 8, 4, 64), 0xA5, dtype=torch.uint8, device=DEV)
    s5.step5_index_summarize(d["k_idx"][:, :T - 8], d["z_idx"][:, :T - 8], 0, d["ln_w"],
                             d["ln_b"], P.EPS, d["rope"], S)
    k_ring = torch.zeros((16, SLOTS, 4, 64), dtype=torch.bfloat16, device=DEV)
    z_ring = torch.zeros_like(k_ring)
    for t in range(T - 8, T - 1):
        k_ring[:, t % SLOTS] = d["k_idx"][:, t]
        z_ring[:, t % SLOTS] = d["z_idx"][:, t]
    rs = d["row_seq"].long()
    k_new = d["k_idx"][rs, T - 1].contiguous()
    z_new = d["z_idx"][rs, T - 1].contiguous()
    ids = torch.full((16, 4, 512), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((16, 4, 512), -7.0, dtype=torch.float32, device=DEV)
    s5.step5_index_append_score_topk(k_new, z_new, k_ring, z_ring, d["ln_w"], d["ln_b"], P.EPS,
                                     d["q_idx"], d["w_head"], d["row_seq"], d["row_pos"], S, ids,
                                     sc, rope=d["rope"], q_norm_w=d["q_norm_w"], q_eps=P.EPS)
    torch.cuda.synchronize()
    P.say("  GPU step done; oracle summaries of 16 sequences")
    O = P.oracle_summary(d)
    return d, S, O, ids, sc


def test_summaries_all_sequences_bitexact(case):
    d, S, O, _, _ = case
    Sg = S.cpu().numpy()
    mism = int((Sg != O).sum())
    P.say(f"  summaries {O.size} codes, mismatches {mism}")
    assert mism == 0


def test_fused_call_selection_all_rows_vs_oracle(case):
    d, _, O, ids, sc = case
    rows = list(range(16))
    osc = P.oracle_scores(d, O, rows)
    ex = P.compare_selection(ids.cpu().numpy(), sc.cpu().numpy(), osc,
                             d["row_pos"].cpu().numpy(), exact=True)
    P.say(f"  16 rows x 4 groups: near-tie excusals {ex}")
    assert ex == 0


def test_plain_selection_equals_fused_call(case):
    d, S, _, ids, sc = case
    ids2, sc2 = P.gpu_select(d, S)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids) and torch.equal(sc2, sc)


def test_attention_all_rows_vs_oracle(case):
    d, _, _, ids, _ = case
    out, lse = P.gpu_attn(d, ids)
    torch.cuda.synchronize()
    oo, ol = P.orc.attend(P.host16(d["q"]), P.host16(d["k_cache"]), P.host16(d["v_cache"]),
                          ids.cpu().numpy(), d["row_seq"].cpu().numpy(),
                          d["row_pos"].cpu().numpy(), P.SCALE)
    e = P.compare_attention(out, lse, oo, ol, "decode16_ctx128k")
    P.say(f"  16 rows: max abs err {e:.3g}")
