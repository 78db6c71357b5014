"""GPU parity of the context sweep: many rows of one sequence (2,048 rows or
more, contexts up to 5,120 regions) are attended tile by tile, 32 rows sharing one pass over the context,
each row masked to its selected regions and its own region up to its
position. Compared with the fp64 oracle (every output element within
2e-3 + 1e-2 |ref|, the log-sum-exp within 2e-3) on sampled rows, and on every
row with the per-row gather path (smaller calls) within twice that.

Also the tiles the sweep leaves to the gather (rows of several sequences in
one tile, rows past its region bound), invalid rows, ragged tiles and
contexts, and cache slots past the rows' positions holding NaN.

Source: TensorFold pull request #903 "Step-5-Preview on one 256 GB Mac"
(indexer commit note: attention over the selected regions plus the row's own
region, causal inside it).
"""
import math

import numpy as np
import pytest
import torch

import parity as P
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1.0 / math.sqrt(128)


def _kv(B, T, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, T, 4, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(B, T, 4, 128, generator=g).to(torch.bfloat16)
    return g, k, v


def _selection(g, pos, valid=None):
    """Per (row, group): min(512, p // 8) distinct candidate ids in random
    order, then -1 (rows marked invalid get -1 throughout)."""
    rows = len(pos)
    sel = np.full((rows, 4, 512), -1, np.int32)
    for r, p in enumerate(pos):
        if valid is not None and not valid[r]:
            continue
        nc = int(p) // 8
        if nc == 0:
            continue
        for gg in range(4):
            ids = torch.randperm(nc, generator=g)[:min(512, nc)].numpy()
            sel[r, gg, :len(ids)] = ids
    return sel


def _gpu(q, k, v, sel, seq, pos, rows_per_call=None):
    rows = q.shape[0]
    out = torch.full((rows, 16, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd, seqd, posd = torch.from_numpy(sel).to(DEV), torch.from_numpy(seq).to(DEV), torch.from_numpy(pos).to(DEV)
    step = rows_per_call or rows
    for a in range(0, rows, step):
        b = min(rows, a + step)
        P.s5.step5_sparse_attn(qd[a:b], kd, vd, sd[a:b], seqd[a:b], posd[a:b], SCALE,
                               out[a:b], lse[a:b])
    torch.cuda.synchronize()
    return out, lse


def _oracle(q, k, v, sel, seq, pos, rows):
    rows = np.asarray(rows)
    return orc.attend(P.host16(q)[rows], P.host16(k), P.host16(v), sel[rows], seq[rows],
                      pos[rows], SCALE)


def _vs_gather(out, lse, q, k, v, sel, seq, pos, where):
    """Every row against the per-row gather path (calls of 512 rows)."""
    og, lg = _gpu(q, k, v, sel, seq, pos, rows_per_call=512)
    a = out.float().cpu().numpy().astype(np.float64)
    b = og.float().cpu().numpy().astype(np.float64)
    err = np.abs(a - b)
    bad = err > 2 * (P.ATOL + P.RTOL * np.abs(b))
    assert not bad.any(), f"{where}: {int(bad.sum())} elements differ from the gather path"
    la, lb = lse.cpu().numpy(), lg.cpu().numpy()
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(la)), where
    assert np.all(np.abs(la[fin] - lb[fin]) <= 4e-3 + 2e-4 * np.abs(lb[fin])), f"{where}: lse"
    return float(err.max())


def test_sweep_prefill_2048_rows_ragged_context():
    """2,048 consecutive rows of one sequence ending at the last slot of an
    8,200-token cache (neither the context nor the last chunk a multiple of
    32 tokens), random selections; then the same call again, bit for bit."""
    T, rows = 8200, 2048
    g, k, v = _kv(1, T, 3)
    q = torch.randn(rows, 16, 128, generator=g).to(torch.bfloat16)
    pos = np.arange(T - rows, T, dtype=np.int64)
    seq = np.zeros(rows, np.int32)
    sel = _selection(g, pos)
    P.say(f"[case] sweep prefill {rows} rows, T={T}")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    pick = sorted(set([0, 1, 31, 32, 33, 63, 500, 1024, 1535, 2015, 2016, 2046, 2047]
                      + torch.randint(0, rows, (12,), generator=g).tolist()))
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "sweep prefill")
    e2 = _vs_gather(out, lse, q, k, v, sel, seq, pos, "sweep prefill")
    P.say(f"  max err vs oracle {e:.2e}, vs gather {e2:.2e}")
    out2, lse2 = _gpu(q, k, v, sel, seq, pos)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)


def test_sweep_peaked_scores():
    """Queries scaled by 12: the scores spread over about +-40 so the
    running max moves often (the rescale path), 2,048 rows."""
    T, rows = 4096, 2048
    g, k, v = _kv(1, T, 8)
    q = (torch.randn(rows, 16, 128, generator=g) * 12).to(torch.bfloat16)
    pos = np.arange(T - rows, T, dtype=np.int64)
    seq = np.zeros(rows, np.int32)
    sel = _selection(g, pos)
    P.say(f"[case] sweep peaked scores {rows} rows")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    pick = [0, 5, 31, 32, 400, 777, 1000, 1023, 2047]
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "peaked")
    e2 = _vs_gather(out, lse, q, k, v, sel, seq, pos, "peaked")
    P.say(f"  max err vs oracle {e:.2e}, vs gather {e2:.2e}")


def test_sweep_nan_past_the_rows():
    """Cache slots past each sequence's last row hold NaN (unwritten slots);
    the rows' own regions end inside those chunks. Two sequences, 1,056 rows
    each (positions 2,000 .. 3,055 and 3,000 .. 4,055 of 4,096 slots)."""
    T = 4096
    g, k, v = _kv(2, T, 12)
    pos = np.concatenate([np.arange(2000, 3056), np.arange(3000, 4056)]).astype(np.int64)
    seq = np.concatenate([np.zeros(1056), np.ones(1056)]).astype(np.int32)
    k[0, 3056:] = float("nan")
    v[0, 3056:] = float("nan")
    k[1, 4056:] = float("nan")
    v[1, 4056:] = float("nan")
    rows = len(pos)
    q = torch.randn(rows, 16, 128, generator=g).to(torch.bfloat16)
    sel = _selection(g, pos)
    P.say(f"[case] sweep NaN past the rows, {rows} rows")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    pick = [0, 31, 1055, 1056, 1057, 2000, 2111]
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "NaN past the rows")
    P.say(f"  max err {e:.2e}")


def test_sweep_nan_in_unselected_regions():
    """The rows select even regions only; the odd regions below every row's
    own region hold NaN in K and V. The gather never reads them; the sweep
    reads whole chunks and must keep them out of scores and outputs. 2,048
    rows at positions 2,048 .. 4,095 of one sequence."""
    T, rows = 4096, 2048
    g, k, v = _kv(1, T, 33)
    pos = np.arange(T - rows, T, dtype=np.int64)
    seq = np.zeros(rows, np.int32)
    q = torch.randn(rows, 16, 128, generator=g).to(torch.bfloat16)
    sel = np.full((rows, 4, 512), -1, np.int32)
    for r, p in enumerate(pos):
        even = np.arange(0, int(p) // 8, 2)
        for gg in range(4):
            pick = even[torch.randperm(len(even), generator=g)[:min(512, len(even))].numpy()]
            sel[r, gg, :len(pick)] = pick
    for j in range(1, (T - rows) // 8, 2):
        k[0, 8 * j:8 * j + 8] = float("nan")
        v[0, 8 * j:8 * j + 8] = float("nan")
    P.say(f"[case] sweep NaN in unselected regions, {rows} rows")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    pick = [0, 1, 31, 32, 500, 1000, 2047]
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "NaN in unselected regions")
    P.say(f"  max err {e:.2e}")


def test_sweep_mixed_tiles_invalid_rows_short_positions():
    """2,054 rows (a ragged last tile of 6) over 3 sequences of 3,000 slots:
    tiles of one sequence at random positions (some below 8: own region only;
    some below 4,096: fewer than 512 candidates), tiles mixing sequences (left
    to the gather), invalid rows (no such sequence, position past the cache)
    inside tiles of one sequence, and a tile of invalid rows only."""
    T, rows = 3000, 2054
    g, k, v = _kv(3, T, 21)
    q = torch.randn(rows, 16, 128, generator=g).to(torch.bfloat16)
    seq = np.zeros(rows, np.int32)
    pos = torch.randint(0, T, (rows,), generator=g).numpy().astype(np.int64)
    for t in range((rows + 31) // 32):
        a, b = 32 * t, min(rows, 32 * t + 32)
        kind = t % 4
        if kind == 0:
            seq[a:b] = 0
        elif kind == 1:
            seq[a:b] = 1
        elif kind == 2:
            seq[a:b] = np.arange(b - a) % 3   # mixed: the gather's rows
        else:
            seq[a:b] = 2
    pos[0:8] = np.arange(8)                  # own region only
    pos[40:48] = [8, 9, 15, 16, 100, 200, 1000, 2999]
    invalid = np.zeros(rows, bool)
    for r in (3, 70, 71, 200, 2053):
        invalid[r] = True
    seq[3], seq[70] = -1, 7
    pos[71], pos[200], pos[2053] = T, T + 5, 10 ** 6
    invalid[32 * 20:32 * 21] = True          # a tile of invalid rows only
    seq[32 * 20:32 * 21] = -1
    sel = _selection(g, np.minimum(pos, T - 1), valid=~invalid)
    P.say(f"[case] sweep mixed tiles, {rows} rows")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert np.all(o[invalid] == 0.0) and np.all(np.isneginf(l[invalid]))
    valid_rows = np.nonzero(~invalid)[0]
    pick = [0, 1, 7, 40, 41, 42, 43, 44, 45, 46, 47, 64, 65, 72, 100, 130, 500, 1000, 2048, 2052]
    pick += valid_rows[torch.randint(0, len(valid_rows), (8,), generator=g).numpy()].tolist()
    pick = sorted(set(r for r in pick if not invalid[r]))
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "mixed tiles")
    e2 = _vs_gather(out, lse, q, k, v, sel, seq, pos, "mixed tiles")
    P.say(f"  max err vs oracle {e:.2e}, vs gather {e2:.2e}")


def test_sweep_region_bound():
    """A 42,000-slot context (5,250 regions): tiles whose own regions reach
    region 5,120 are left to the gather, the others are swept; 2,048 rows at
    positions 39,000 .. 40,023 and 40,976 .. 41,999."""
    T = 42000
    g, k, v = _kv(1, T, 30)
    pos = np.concatenate([np.arange(39000, 40024), np.arange(40976, 42000)]).astype(np.int64)
    seq = np.zeros(len(pos), np.int32)
    rows = len(pos)
    q = torch.randn(rows, 16, 128, generator=g).to(torch.bfloat16)
    sel = _selection(g, pos)
    P.say(f"[case] sweep region bound, {rows} rows, T={T}")
    out, lse = _gpu(q, k, v, sel, seq, pos)
    pick = [0, 1023, 1024, 1040, 1055, 1056, 1057, 2000, 2047]
    oo, ol = _oracle(q, k, v, sel, seq, pos, pick)
    e = P.compare_attention(out[pick], lse[pick], oo, ol, "region bound")
    P.say(f"  max err {e:.2e}")
