"""GPU parity of the sparse attention for the other query-head geometries:
8 or 16 query heads per KV head, 128- or 192-dim heads (Step-5's own layers
have 16 heads per KV group of 192 dims; vLLM's geometry rules allow 4, 8 or
16). The fp64 oracle runs on the GPU's own inputs and selections; every
output element within 2e-3 + 1e-2 |ref|, the log-sum-exp within 2e-3.

Sources: TensorFold pull request #903 "Step-5-Preview on one 256 GB Mac"
(attention notes: the group's 16 query heads over 192 dims); vLLM
"vllm.models.step5.nvidia.model" (_validate_step5_dsa_parallel_geometry).
"""
import math

import numpy as np
import pytest
import torch

import parity as P
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"
GEOMS = [(32, 128), (64, 128), (16, 192), (32, 192), (64, 192)]


def _inputs(Hq, D, B, T, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, T, 4, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, T, 4, D, generator=g).to(torch.bfloat16)
    return g, k, v


def _random_selection(g, pos, ncap=512):
    """Per (row, group): min(512, p // 8) distinct candidate ids in random
    order, then -1."""
    rows = len(pos)
    sel = np.full((rows, 4, ncap), -1, np.int32)
    for r, p in enumerate(pos):
        nc = int(p) // 8
        for gg in range(4):
            ids = torch.randperm(nc, generator=g)[:min(ncap, nc)].numpy() if nc else np.zeros(0)
            sel[r, gg, :len(ids)] = ids
    return sel


def _run(Hq, D, q, k, v, sel, seq, pos):
    rows = q.shape[0]
    out = torch.full((rows, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device=DEV)
    P.s5.step5_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                           torch.from_numpy(seq).to(DEV), torch.from_numpy(pos).to(DEV),
                           1.0 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    oo, ol = orc.attend(P.host16(q), P.host16(k), P.host16(v), sel, seq, pos, 1.0 / math.sqrt(D))
    return out, lse, oo, ol


@pytest.mark.parametrize("Hq,D", GEOMS)
def test_geometry_decode_split(Hq, D):
    """4 decode rows of 4 sequences at position 5,999 (749 candidates, 512
    selected): the split path and its merge."""
    g, k, v = _inputs(Hq, D, 4, 6000, 17)
    q = torch.randn(4, Hq, D, generator=g).to(torch.bfloat16)
    pos = np.full(4, 5999, np.int64)
    seq = np.arange(4, dtype=np.int32)
    sel = _random_selection(g, pos)
    P.say(f"[case] geometry Hq={Hq} D={D} decode 4 x 6000")
    out, lse, oo, ol = _run(Hq, D, q, k, v, sel, seq, pos)
    err = P.compare_attention(out, lse, oo, ol, f"Hq={Hq} D={D}")
    P.say(f"  max err {err:.2e}")


@pytest.mark.parametrize("Hq,D", [(64, 192), (32, 128)])
def test_geometry_all_selected_equals_dense(Hq, D):
    """3,000-token contexts: 374 candidates, all selected, so the sparse
    attention is the dense causal attention; rows at positions 2,999, 7
    (own region only) and 8 (one candidate) of three sequences."""
    g, k, v = _inputs(Hq, D, 3, 3000, 41)
    q = torch.randn(3, Hq, D, generator=g).to(torch.bfloat16)
    pos = np.array([2999, 7, 8], np.int64)
    seq = np.arange(3, dtype=np.int32)
    sel = _random_selection(g, pos)
    P.say(f"[case] geometry Hq={Hq} D={D} all selected")
    out, lse, oo, ol = _run(Hq, D, q, k, v, sel, seq, pos)
    P.compare_attention(out, lse, oo, ol, f"Hq={Hq} D={D} dense")
    # the oracle's sparse attention equals plain dense causal attention here
    qf = q.double()
    kf, vf = k.double(), v.double()
    for r in range(3):
        p = int(pos[r])
        for h in (0, Hq - 1):
            gg = h // (Hq // 4)
            s = (kf[r, :p + 1, gg] @ qf[r, h]) / math.sqrt(D)
            w = torch.softmax(s, 0)
            assert np.allclose(oo[r, h], (w @ vf[r, :p + 1, gg]).numpy(), atol=1e-9)


@pytest.mark.parametrize("Hq,D", [(64, 192), (32, 128)])
def test_geometry_prefill_unsplit(Hq, D):
    """300 rows of one 4,096-token sequence (positions 3,796 .. 4,095): enough
    units to run unsplit, regions visited in id order."""
    rows = 300
    g, k, v = _inputs(Hq, D, 1, 4096, 5)
    q = torch.randn(rows, Hq, D, generator=g).to(torch.bfloat16)
    pos = np.arange(4096 - rows, 4096, dtype=np.int64)
    seq = np.zeros(rows, np.int32)
    sel = _random_selection(g, pos)
    P.say(f"[case] geometry Hq={Hq} D={D} prefill {rows} rows")
    out, lse, oo, ol = _run(Hq, D, q, k, v, sel, seq, pos)
    P.compare_attention(out, lse, oo, ol, f"Hq={Hq} D={D} prefill")


def test_geometry_invalid_rows_write_zeros():
    """Rows whose sequence or position is out of range attend to nothing:
    zero output, log-sum-exp -inf (both paths: split and unsplit)."""
    Hq, D = 64, 192
    g, k, v = _inputs(Hq, D, 2, 64, 9)
    for rows in (2, 300):
        q = torch.randn(rows, Hq, D, generator=g).to(torch.bfloat16)
        seq = np.full(rows, 0, np.int32)
        pos = np.full(rows, 40, np.int64)
        seq[0] = 7          # no such sequence
        pos[1] = 64         # past the cache
        sel = _random_selection(g, np.minimum(pos, 63))
        out = torch.full((rows, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device=DEV)
        P.s5.step5_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(sel).to(DEV),
                               torch.from_numpy(seq).to(DEV), torch.from_numpy(pos).to(DEV),
                               1.0 / math.sqrt(D), out, lse)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        assert np.all(o[:2] == 0.0)
        assert np.all(np.isneginf(lse.cpu().numpy()[:2]))
        assert np.all(np.isfinite(o[2:]))
