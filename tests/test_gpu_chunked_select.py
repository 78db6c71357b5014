"""GPU parity of the decode selection when a unit's candidates are cut into
several chunks (more than 16,384 regions, up to 64 rows): the exact scorer
leaves per block the best key of every 32 candidates, the selection takes
from them a bound of each unit's 512th best score, every chunk keeps only
the candidates that reach it (at most its best 512), and the last chunk to
arrive sorts the union. Ids and scores must equal the oracle's bit for bit.

Cases: random finite e4m3 codes and tie-heavy codes over 40,000 regions
(3 chunks) with rows whose candidate counts straddle chunk and block
borders, and invalid rows; one row over the largest summary accepted
(524,288 regions, 32 chunks); every score equal (all candidates tie, so
each chunk has far more than 512 at the bound); and a workspace that holds
garbage, then the keys of an earlier call with longer rows.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_indexer_amd as s5
import workloads as W
import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _draw(kind, g):
    if kind == "random":
        def draw(shape):
            c = torch.randint(0, 0x7F, shape, generator=g, dtype=torch.int32)   # 0x7F is NaN
            return (c | (torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
        return draw, torch.rand(16, generator=g)
    tie = torch.tensor(W.TIE_CODES, dtype=torch.uint8)
    return (lambda shape: tie[torch.randint(0, 8, shape, generator=g)],
            torch.arange(1, 17, dtype=torch.float32) / 16)


def _select(d, S, ws=None):
    rows = d["rows"]
    ids = torch.full((rows, 4, 512), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((rows, 4, 512), -7.0, dtype=torch.float32, device=DEV)
    s5.step5_index_score_topk(d["q8"], d["w_head"], d["row_seq"], d["row_pos"], S, ids, sc,
                              q_is_e4m3=True, workspace=ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def _check(d, S, ids, sc, good, bad=()):
    osc = P.oracle_scores(d, P.host8(S), list(good))
    pos = d["row_pos"].cpu().numpy()[list(good)]
    ex = P.compare_selection(ids[list(good)], sc[list(good)], osc, pos, exact=True)
    assert ex == 0
    for r in bad:
        assert np.all(ids[r] == -1) and np.all(sc[r] == 0), r


def _rows_case(kind, seed, ncands, R):
    g = torch.Generator().manual_seed(seed)
    draw, w = _draw(kind, g)
    B = len(ncands)
    pos = [8 * c + (5 * i) % 8 for i, c in enumerate(ncands)]
    seq = list(range(B))
    # invalid rows: no sequence, a sequence past the batch, a position past the summary
    seq += [-1, B, 2]
    pos += [8 * 30000, 8 * 30000, 8 * R + 8]
    rows = len(seq)
    d = {"rows": rows, "q8": draw((rows, 16, 64)).to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.tensor(seq, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor(pos, dtype=torch.int64, device=DEV)}
    return d, draw((B, R, 4, 64)).to(DEV), B


NCANDS = [0, 1, 300, 511, 512, 513, 13375, 13376, 13377, 20000, 26751, 39999]


@pytest.mark.parametrize("kind", ["random", "tie_heavy"])
def test_chunked_select_rows_over_40000_regions(kind):
    R = 40000
    d, S, B = _rows_case(kind, 31 if kind == "random" else 32, NCANDS, R)
    P.say(f"[case] chunked select {kind}: {d['rows']} rows over {R} regions")
    ids, sc = _select(d, S)
    _check(d, S, ids, sc, range(B), range(B, d["rows"]))


def test_chunked_select_largest_summary():
    """One row over 524,288 regions (32 chunks): the scorer's keys take more
    than one pass of the selection's threshold loads."""
    R = 524288
    g = torch.Generator().manual_seed(33)
    draw, w = _draw("random", g)
    d = {"rows": 1, "q8": draw((1, 16, 64)).to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.zeros(1, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor([8 * R - 1], dtype=torch.int64, device=DEV)}
    S = draw((1, R, 4, 64)).to(DEV)
    P.say(f"[case] chunked select: 1 row over {R} regions")
    ids, sc = _select(d, S)
    _check(d, S, ids, sc, [0])


def test_chunked_select_every_score_equal():
    """Every candidate has the same score: each chunk keeps its 512 smallest
    ids, the union is sorted by id, and the selection is regions 0..511."""
    R = 131072
    code = 0x38  # 1.0 in e4m3
    d = {"rows": 1, "q8": torch.full((1, 16, 64), code, dtype=torch.uint8, device=DEV),
         "w_head": (torch.arange(1, 17, dtype=torch.float32) / 16).to(DEV),
         "row_seq": torch.zeros(1, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor([8 * R - 1], dtype=torch.int64, device=DEV)}
    S = torch.full((1, R, 4, 64), code, dtype=torch.uint8, device=DEV)
    P.say(f"[case] chunked select: every score equal over {R} regions")
    ids, sc = _select(d, S)
    assert np.array_equal(ids[0], np.tile(np.arange(512, dtype=np.int32), (4, 1)))
    _check(d, S, ids, sc, [0])


def test_chunked_select_workspace_garbage_then_stale_keys():
    """The workspace starts as 0xFF bytes (the largest key in every slot the
    scorer does not write this call); a second call on the same workspace has
    shorter rows, so the blocks past them hold the first call's keys."""
    R = 40000
    d, S, B = _rows_case("random", 34, NCANDS, R)
    nb = s5.step5_index_score_topk_workspace(d["rows"], R)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)
    P.say(f"[case] chunked select, garbage workspace: {d['rows']} rows over {R} regions")
    ids, sc = _select(d, S, ws)
    _check(d, S, ids, sc, range(B), range(B, d["rows"]))
    short = [max(0, c // 3) for c in NCANDS]
    d2, S2, _ = _rows_case("random", 35, short, R)
    P.say(f"[case] chunked select, stale keys: rows of {short} candidates")
    ids, sc = _select(d2, S2, ws)
    _check(d2, S2, ids, sc, range(B), range(B, d2["rows"]))
