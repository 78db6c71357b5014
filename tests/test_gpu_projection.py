"""GPU parity of the fused projection (one product hidden @ W^T whose columns
are split into q, k, v, index_q, index_k, index_z and the gate) against the
fp64 oracle.

Tolerance, from the arithmetic: each output is a sum of bf16 products
accumulated in fp32 (at most 256 roundings of a partial sum, each within
2^-24 of it, the partial sums bounded by S = sum_k |h_k w_k|), rounded once
to bf16 (within 2^-9 of the value). So |gpu - ref| <= 2^-8 |ref| + 2^-16 S,
both terms with a factor 2 to spare. Where the weight is one-hot the sums are
exact and the outputs must equal the hidden values bit for bit.

Source: vLLM "vllm.models.step5.nvidia.model", Step5FusedQKVIndexerLinear
(forward: one hidden @ W^T; split_indexer: the column blocks).
"""
import numpy as np
import pytest
import torch

import parity as P
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(rows, H, N, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(rows, H, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    return g, h, w


def _outs(rows, widths, pad=0, fill=-7.0):
    """Outputs as [rows, width] views of [rows, width + pad] buffers filled
    with a sentinel (so writes past a part's width can be seen)."""
    bufs = [torch.full((rows, wd + pad), fill, dtype=torch.bfloat16, device=DEV) for wd in widths]
    return bufs, [b[:, :wd] for b, wd in zip(bufs, widths)]


def _run(h, w, widths, pad=0, hidden_pad=0, **kw):
    rows, H = h.shape
    hd = torch.zeros(rows, H + hidden_pad, dtype=torch.bfloat16, device=DEV)
    hd[:, :H] = h.to(DEV)
    bufs, outs = _outs(rows, widths, pad)
    P.s5.step5_qkv_index_project(hd[:, :H], w.to(DEV), outs, gate_size=widths[6], **kw)
    torch.cuda.synchronize()
    return bufs, outs


def _compare(outs, h, w, widths, rows_idx, where):
    """Every element of the given rows against the oracle."""
    rows_idx = np.asarray(rows_idx)
    hh = P.host16(h)[rows_idx]
    ref, _ = orc.project(hh, P.host16(w), widths)
    S = np.abs(orc.bf16_to_f32(hh).astype(np.float64)) @ np.abs(orc.bf16_to_f32(P.host16(w)).astype(np.float64)).T
    got = np.concatenate([o.float().cpu().numpy()[rows_idx] for o in outs if o.shape[1]], axis=1)
    err = np.abs(got.astype(np.float64) - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * S
    bad = err > bound
    assert not bad.any(), (f"{where}: {int(bad.sum())} of {bad.size} outside the bound; "
                           f"max err {err.max():.3g}")
    return float(err.max()), float((err / np.maximum(bound, 1e-30)).max())


def test_project_decode_16_rows_every_element():
    """16 rows (the decode shape), hidden 4,096, the layer's 4,624 columns."""
    widths = orc.proj_sizes()
    _, h, w = _inputs(16, 4096, sum(widths), 1)
    P.say("[case] projection 16 x 4096 -> 4624")
    _, outs = _run(h, w, widths)
    e, r = _compare(outs, h, w, widths, range(16), "decode")
    P.say(f"  max err {e:.3g} ({r:.2f} of the bound)")


def test_project_prefill_2048_rows_sampled():
    """2,048 rows (a prompt chunk) on the tiled kernel; 40 rows compared,
    among them the first and last of tiles; then the same call again, bit for
    bit."""
    widths = orc.proj_sizes()
    g, h, w = _inputs(2048, 4096, sum(widths), 2)
    P.say("[case] projection 2048 x 4096 -> 4624")
    _, outs = _run(h, w, widths)
    pick = sorted(set([0, 1, 31, 32, 63, 64, 65, 127, 128, 1000, 1023, 1024, 2046, 2047] +
                      torch.randint(0, 2048, (26,), generator=g).tolist()))
    e, r = _compare(outs, h, w, widths, pick, "prefill")
    P.say(f"  max err {e:.3g} ({r:.2f} of the bound)")
    _, outs2 = _run(h, w, widths)
    for a, b in zip(outs, outs2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("rows", [1, 15, 17, 63, 64, 65, 129, 200])
def test_project_ragged_rows(rows):
    """Row counts around both kernels' tiles (16 and 64 rows), hidden 512."""
    widths = orc.proj_sizes()
    _, h, w = _inputs(rows, 512, sum(widths), 10 + rows)
    P.say(f"[case] projection {rows} x 512")
    bufs, outs = _run(h, w, widths, pad=32)
    _compare(outs, h, w, widths, range(rows), f"rows={rows}")
    for b, wd in zip(bufs, widths):
        assert torch.all(b[:, wd:].float() == -7.0), "wrote past a part's width"


@pytest.mark.parametrize("rows", [16, 200])
def test_project_one_hot_weight_is_exact(rows):
    """Each weight row one-hot at a column of hidden: every output is that
    hidden value, bit for bit (both kernels)."""
    widths = orc.proj_sizes()
    N, H = sum(widths), 1024
    g = torch.Generator().manual_seed(5)
    h = (torch.randn(rows, H, generator=g) * 3).to(torch.bfloat16)
    col = torch.randint(0, H, (N,), generator=g)
    w = torch.zeros(N, H)
    w[torch.arange(N), col] = 1.0
    P.say(f"[case] projection one-hot weight, {rows} rows")
    _, outs = _run(h, w.to(torch.bfloat16), widths)
    got = torch.cat([o.cpu() for o in outs], dim=1)
    assert torch.equal(got.view(torch.int16), h[:, col].view(torch.int16))


def test_project_strided_hidden_and_outputs_gate_zero():
    """hidden rows with a stride past their width, every output a view into a
    wider buffer, no gate (six outputs)."""
    widths = orc.proj_sizes()[:6] + (0,)
    _, h, w = _inputs(96, 1024, sum(widths), 7)
    P.say("[case] projection strided, gate 0")
    bufs, outs = _run(h, w, widths, pad=64, hidden_pad=128)
    _compare(outs, h, w, widths, range(96), "strided")
    for b, wd in zip(bufs, widths):
        assert torch.all(b[:, wd:].float() == -7.0)


def test_project_64_heads_of_192():
    """Step-5's own attention shape: 16 query heads per KV head of 192 dims
    (q 12,288 columns, k and v 768), a gate per query head (64)."""
    widths = orc.proj_sizes(q_heads=64, head_dim=192, gate=64)
    _, h, w = _inputs(70, 512, sum(widths), 9)
    P.say("[case] projection 64 x 192 geometry")
    _, outs = _run(h, w, widths, q_heads=64, head_dim=192)
    _compare(outs, h, w, widths, range(70), "64x192")


def test_project_wide_tiles_64_heads_of_192():
    """The tiled kernel on Step-5's own shape: 300 rows (two full 128-row
    tiles and a ragged one), 15,424 columns (48 full 320-column tiles and a
    last one of 64), hidden 512; 24 rows compared, among them each tile's
    first and last."""
    widths = orc.proj_sizes(q_heads=64, head_dim=192, gate=64)
    g, h, w = _inputs(300, 512, sum(widths), 12)
    P.say("[case] projection 300 rows, 64 x 192 geometry (tiled kernel)")
    bufs, outs = _run(h, w, widths, pad=16, q_heads=64, head_dim=192)
    pick = sorted(set([0, 1, 127, 128, 255, 256, 257, 298, 299] +
                      torch.randint(0, 300, (15,), generator=g).tolist()))
    _compare(outs, h, w, widths, pick, "wide 64x192")
    for b, wd in zip(bufs, widths):
        assert torch.all(b[:, wd:].float() == -7.0), "wrote past a part's width"
