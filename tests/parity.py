"""Helpers of the GPU parity tests: run the HIP path (through the C ABI's
Python binding) and the CPU oracle on the same input bytes, and compare them
under the path's acceptance rules:

  summaries   e4m3 codes bit-exact;
  selections  region ids and their scores bit-exact position by position
              (the GPU rescores every possible member exactly). The
              comparison can also excuse near-ties (oracle scores of the two
              ids within 1e-6 of the last kept score) and count them; the
              tests run it strict, with no excusal allowed;
  attention   |gpu - oracle| <= 2e-3 + 1e-2 |oracle| element by element, the
              oracle run in fp64 on the GPU's own selection.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import long_context_sparse_indexer_amd as s5  # noqa: E402
import workloads as W  # noqa: E402
from oracle import oracle as orc  # noqa: E402

EPS = W.NORM_EPS
SCALE = 1.0 / math.sqrt(W.HEAD_DIM)
ATOL, RTOL = 2e-3, 1e-2
TIE_REL = 1e-6


def say(*a):
    print(*a, flush=True)


def host16(t):
    return W.bits16(t)


def host8(t):
    return W.bits8(t)


# ---- GPU path -------------------------------------------------------------

def gpu_summary(d, dev="cuda", k="k_idx", z="z_idx", t0=0, R_cap=None):
    kk, zz = d[k].to(dev), d[z].to(dev)
    B, T = kk.shape[0], kk.shape[1]
    R_cap = R_cap or (t0 + T) // 8
    S = torch.zeros((B, R_cap, 4, 64), dtype=torch.uint8, device=dev)
    s5.step5_index_summarize(kk, zz, t0, d["ln_w"].to(dev), d["ln_b"].to(dev), EPS,
                             d["rope"].to(dev), S)
    return S


def gpu_select(d, S, dev="cuda"):
    rows = d["rows"]
    ids = torch.full((rows, 4, 512), -7, dtype=torch.int32, device=dev)
    sc = torch.full((rows, 4, 512), -7.0, dtype=torch.float32, device=dev)
    if "q8" in d:
        s5.step5_index_score_topk(d["q8"].to(dev), d["w_head"].to(dev), d["row_seq"].to(dev),
                                  d["row_pos"].to(dev), S, ids, sc, q_is_e4m3=True)
    else:
        s5.step5_index_score_topk(d["q_idx"].to(dev), d["w_head"].to(dev), d["row_seq"].to(dev),
                                  d["row_pos"].to(dev), S, ids, sc, q_norm_w=d["q_norm_w"].to(dev),
                                  q_eps=EPS, rope=d["rope"].to(dev))
    return ids, sc


def gpu_attn(d, ids, dev="cuda"):
    rows = d["rows"]
    out = torch.full((rows, 16, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((rows, 16), float("nan"), dtype=torch.float32, device=dev)
    s5.step5_sparse_attn(d["q"].to(dev), d["k_cache"].to(dev), d["v_cache"].to(dev), ids,
                         d["row_seq"].to(dev), d["row_pos"].to(dev), SCALE, out, lse)
    return out, lse


# ---- oracle path ------------------------------------------------------------

def oracle_summary(d, k="k_idx", z="z_idx", t0=0, seqs=None, R_cap=None):
    k16, z16 = host16(d[k]), host16(d[z])
    if seqs is not None:
        k16, z16 = k16[seqs], z16[seqs]
    return orc.summarize(k16, z16, t0, d["ln_w"].cpu().numpy(), d["ln_b"].cpu().numpy(), EPS,
                         host16(d["rope"]), R_cap=R_cap)


def oracle_q8(d, rows=None):
    if "q8" in d:
        q8 = host8(d["q8"])
        return q8 if rows is None else q8[rows]
    q16 = host16(d["q_idx"])
    pos = d["row_pos"].cpu().numpy()
    if rows is not None:
        q16, pos = q16[rows], pos[rows]
    return orc.q_prep(q16, d["q_norm_w"].cpu().numpy(), EPS, host16(d["rope"]), pos)


def oracle_scores(d, summary_np, rows, seq_map=None):
    """All candidate scores [len(rows), 4, R_cap] of the given rows, the rows'
    sequences renumbered by seq_map into the summary array given."""
    q8 = oracle_q8(d, rows)
    seq = d["row_seq"].cpu().numpy()[rows].astype(np.int32)
    if seq_map is not None:
        seq = np.array([seq_map[s] for s in seq], np.int32)
    pos = d["row_pos"].cpu().numpy()[rows]
    w = d["w_head"].cpu().numpy()
    return orc.score(q8, w, seq, pos, summary_np)


# ---- comparisons ------------------------------------------------------------

def compare_selection(gids, gsc, oscores, pos, topk=512, exact=True):
    """gids/gsc: GPU ids and scores [n, 4, topk]; oscores: oracle scores of all
    candidates [n, 4, R_cap]; pos: positions [n]. Returns the excusal count;
    raises AssertionError on a failure."""
    oids, osel = orc.select(oscores, pos, topk)
    excused = 0
    for r in range(gids.shape[0]):
        nc = int(pos[r]) // 8
        K = min(topk, nc)
        for g in range(4):
            gi, oi = gids[r, g], oids[r, g]
            assert np.all(gi[K:] == -1) and np.all(oi[K:] == -1), (r, g, "padding")
            assert np.all(gsc[r, g, K:] == 0.0), (r, g, "score padding")
            sel = gi[:K]
            assert np.all((sel >= 0) & (sel < nc)), (r, g, "id range")
            assert len(np.unique(sel)) == K, (r, g, "duplicate ids")
            s = oscores[r, g]
            bound = TIE_REL * max(abs(float(s[oi[K - 1]])), np.finfo(np.float32).tiny) if K else 0
            for i in np.nonzero(gi[:K] != oi[:K])[0]:
                diff = abs(float(s[gi[i]]) - float(s[oi[i]]))
                if exact or diff >= bound:
                    raise AssertionError(
                        f"row {r} group {g} pos {i}: gpu id {gi[i]} (oracle score {s[gi[i]]!r}) "
                        f"vs oracle id {oi[i]} ({s[oi[i]]!r}); bound {bound:.3g}")
                excused += 1
            # GPU scores of its picks against the oracle's scores of the same ids
            ref = s[sel].astype(np.float64)
            got = gsc[r, g, :K].astype(np.float64)
            if exact:
                assert np.array_equal(got, ref), (r, g, "scores")
            else:
                assert np.all(np.abs(got - ref) <= 1e-4 * (1.0 + np.abs(ref))), (r, g, "scores")
    return excused


def compare_attention(out_g, lse_g, out_o, lse_o, where=""):
    og = out_g.float().cpu().numpy().astype(np.float64)
    err = np.abs(og - out_o)
    bad = err > ATOL + RTOL * np.abs(out_o)
    assert not bad.any(), (f"{where}: {int(bad.sum())} elements out of tolerance; "
                           f"max err {err.max():.3g}")
    lg = lse_g.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lg - lse_o) <= 2e-3 + 1e-4 * np.abs(lse_o)), f"{where}: lse"
    return float(err.max())
