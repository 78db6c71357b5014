"""GPU parity of the decode selection at shapes the workload tests do not
reach: up to 64 rows over 5,000 and 16,384 regions, e4m3 query and summaries
drawn directly. Ids and scores must equal the oracle's bit for bit (no
near-tie excusal).

Cases: rows with 0, 1, 511, 512, 513, 1,023, 1,024, 1,025 candidates and the
full range, invalid rows (no sequence, a sequence past the batch, a position
past the summary), every finite e4m3 code at random, and tie-heavy codes
from {+-1/4 .. +-2} (many exact ties around the 512th score).
"""
import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("kind", ["random", "tie_heavy"])
def test_decode_select_edge_rows(kind):
    B, R = 12, 5000
    g = torch.Generator().manual_seed(7 if kind == "random" else 8)
    draw, w = _draw(kind, g)
    ncands = [0, 1, 511, 512, 513, 1023, 1024, 1025, 2777, 4999, 4999, 4999]
    pos = [8 * c + (3 * i) % 8 for i, c in enumerate(ncands)]
    seq = list(range(B))
    # invalid rows: no sequence, a sequence past the batch, a position past the summary
    seq += [-1, B, 3]
    pos += [8 * 4000, 8 * 4000, 8 * R + 8]
    rows = len(seq)
    d = {"rows": rows, "q8": draw((rows, 16, 64)).to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.tensor(seq, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor(pos, dtype=torch.int64, device=DEV)}
    S = draw((B, R, 4, 64)).to(DEV)
    P.say(f"[case] decode select {kind}: {rows} rows over {R} regions")
    ids, sc = P.gpu_select(d, S)
    torch.cuda.synchronize()
    ids_h, sc_h = ids.cpu().numpy(), sc.cpu().numpy()
    good = list(range(B))
    osc = P.oracle_scores(d, P.host8(S), good)
    ex = P.compare_selection(ids_h[good], sc_h[good], osc, np.array(pos)[good], exact=True)
    assert ex == 0
    for bad in range(B, rows):
        assert np.all(ids_h[bad] == -1) and np.all(sc_h[bad] == 0), bad


def test_decode_select_tie_heavy_16_rows_16384_regions():
    """16 rows over 16,384 regions each, tie-heavy codes: many exact ties
    around the 512th score, ordered by region id."""
    rows, R = 16, 16384
    g = torch.Generator().manual_seed(9)
    draw, w = _draw("tie_heavy", g)
    d = {"rows": rows, "q8": draw((rows, 16, 64)).to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.arange(rows, dtype=torch.int32, device=DEV),
         "row_pos": torch.full((rows,), 8 * R - 1, dtype=torch.int64, device=DEV)}
    S = draw((rows, R, 4, 64)).to(DEV)
    P.say(f"[case] decode select tie-heavy: {rows} rows x {R} regions")
    ids, sc = P.gpu_select(d, S)
    torch.cuda.synchronize()
    osc = P.oracle_scores(d, P.host8(S), list(range(rows)))
    ex = P.compare_selection(ids.cpu().numpy(), sc.cpu().numpy(), osc,
                             d["row_pos"].cpu().numpy(), exact=True)
    assert ex == 0


@pytest.mark.parametrize("R", [16384, 40000])
def test_decode_select_zero_score_ties(R):
    """Many candidates tie at the 512th score: candidates whose dots are all
    negative score exactly 0 after relu. Rows with 400 positive scores among
    2,000 candidates, none among all R, and 600 among all R: more than 1,024
    candidates reach the threshold, and the 0-score ties must go by smaller
    id (one selection chunk at 16,384 regions, several at 40,000)."""
    g = torch.Generator().manual_seed(12)
    npos = [(2000, 400), (R - 1, 0), (R - 1, 600)]
    rows = len(npos)
    S = (0x81 + torch.randint(0, 0x7E - 0x00, (rows, R, 4, 64), generator=g)).to(torch.uint8)
    for r, (nc, npositive) in enumerate(npos):
        pick = torch.randperm(nc, generator=g)[:npositive]
        S[r, pick] = (1 + torch.randint(0, 0x7E, (npositive, 4, 64), generator=g)).to(torch.uint8)
    d = {"rows": rows, "q8": torch.full((rows, 16, 64), 0x38, dtype=torch.uint8).to(DEV),
         "w_head": (torch.rand(16, generator=g) + 0.5).to(DEV),
         "row_seq": torch.arange(rows, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor([8 * nc + 7 for nc, _ in npos], dtype=torch.int64, device=DEV)}
    S = S.to(DEV)
    P.say(f"[case] decode select, zero-score ties: {rows} rows over {R} regions")
    ids, sc = P.gpu_select(d, S)
    torch.cuda.synchronize()
    osc = P.oracle_scores(d, P.host8(S), list(range(rows)))
    ex = P.compare_selection(ids.cpu().numpy(), sc.cpu().numpy(), osc,
                             d["row_pos"].cpu().numpy(), exact=True)
    assert ex == 0


def test_fused_select_mixed_row_blocks():
    """More than 64 rows over at most 4,096 regions take the fused interval
    selection, which scores 4 consecutive rows at once when they share a
    sequence and row by row otherwise. 70 rows (the last block of 4 is
    partial): blocks of one sequence at consecutive positions (as a prompt
    chunk), blocks mixing sequences, rows with 0, 1, 511, 512 and 513
    candidates, and invalid rows (no sequence, a sequence past the batch, a
    position past the summary). Ids and scores equal the oracle's."""
    B, R = 6, 3000
    g = torch.Generator().manual_seed(13)
    draw, w = _draw("random", g)
    seq, pos = [], []
    for b in range(8):              # blocks of one sequence, consecutive positions
        s = b % 4
        p0 = 8 * (1200 + 150 * b) + 3
        seq += [s] * 4
        pos += [p0 + i for i in range(4)]
    for b in range(6):              # blocks mixing sequences and candidate counts
        seq += [4, 5, b % 4, (b + 1) % 4]
        pos += [8 * 2999 + 2, 8 * (100 * b + 7), 8 * 512 + b, 8 * (2000 + b) + 7]
    seq += [0, 1, 2, 3, 4, 5, 0, 1, 2, 3, 2, 5]  # edge counts, then invalid rows
    pos += [0, 8 * 1, 8 * 511 + 5, 8 * 512, 8 * 513 + 7, 8 * 2999 + 7, 8 * 2800, 8 * 17, 8 * 2000,
            8 * 640, 8 * 1500 + 1, 8 * 300]
    seq += [-1, B]
    pos += [8 * 1000, 8 * 1000]
    seq[-4], pos[-4] = 3, 8 * R + 8   # a position past the summary
    rows = len(seq)
    assert rows == 70
    d = {"rows": rows, "q8": draw((rows, 16, 64)).to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.tensor(seq, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor(pos, dtype=torch.int64, device=DEV)}
    S = draw((B, R, 4, 64)).to(DEV)
    P.say(f"[case] fused selection, mixed 4-row blocks: {rows} rows over {R} regions")
    ids, sc = P.gpu_select(d, S)
    torch.cuda.synchronize()
    ids_h, sc_h = ids.cpu().numpy(), sc.cpu().numpy()
    bad = [r for r in range(rows) if not (0 <= seq[r] < B and pos[r] // 8 <= R)]
    good = [r for r in range(rows) if r not in bad]
    osc = P.oracle_scores(d, P.host8(S), good)
    ex = P.compare_selection(ids_h[good], sc_h[good], osc, np.array(pos)[good], exact=True)
    assert ex == 0
    for r in bad:
        assert np.all(ids_h[r] == -1) and np.all(sc_h[r] == 0), r


@pytest.mark.parametrize("kind", ["every_score_equal", "tie_heavy"])
def test_fused_select_many_survivors(kind):
    """The fused interval selection when one unit's survivors outnumber
    1,024: every score equal (all 2,999 candidates of a row tie at the
    threshold, so the unit is redone by the whole workgroup, cut and radix
    selected, and keeps regions 0..511), and tie-heavy codes (8 distinct
    values). 68 rows of 4 sequences over 3,000 regions, rows of one block
    sharing a sequence. Ids and scores equal the oracle's."""
    B, R, rows = 4, 3000, 68
    g = torch.Generator().manual_seed(17)
    seq = [(r // 4) % B for r in range(rows)]
    pos = [8 * 2999 + (r % 8) for r in range(rows)]
    if kind == "every_score_equal":
        code = 0x38  # 1.0 in e4m3
        q8 = torch.full((rows, 16, 64), code, dtype=torch.uint8)
        S = torch.full((B, R, 4, 64), code, dtype=torch.uint8)
        w = torch.arange(1, 17, dtype=torch.float32) / 16
    else:
        draw, w = _draw("tie_heavy", g)
        q8, S = draw((rows, 16, 64)), draw((B, R, 4, 64))
    d = {"rows": rows, "q8": q8.to(DEV), "w_head": w.to(DEV),
         "row_seq": torch.tensor(seq, dtype=torch.int32, device=DEV),
         "row_pos": torch.tensor(pos, dtype=torch.int64, device=DEV)}
    S = S.to(DEV)
    P.say(f"[case] fused selection, many survivors ({kind}): {rows} rows over {R} regions")
    ids, sc = P.gpu_select(d, S)
    torch.cuda.synchronize()
    ids_h, sc_h = ids.cpu().numpy(), sc.cpu().numpy()
    if kind == "every_score_equal":
        assert np.array_equal(ids_h, np.tile(np.arange(512, dtype=np.int32), (rows, 4, 1)))
    good = list(range(rows))
    osc = P.oracle_scores(d, P.host8(S), good)
    ex = P.compare_selection(ids_h, sc_h, osc, np.array(pos), exact=True)
    assert ex == 0
