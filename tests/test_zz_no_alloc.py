"""step5_sparse_attn_noalloc (the allocation-free entry point, for callers
that cannot allocate device memory) against step5_sparse_attn: the same
output and log-sum-exp bit for bit, on two calls in a row, the second with
fewer rows, for the 4-heads x 128 attention and the 16-heads x 192 one (each
needs split states in the static scratch at these row counts)."""
import math

import pytest
import torch

import long_context_sparse_indexer_amd as s5

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(rows, Hq, D, T, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    B = rows
    q = torch.randn((rows, Hq, D), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, T, 4, D), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, T, 4, D), generator=g, device=DEV).to(torch.bfloat16)
    seq = torch.arange(rows, dtype=torch.int32, device=DEV)
    pos = T - 1 - torch.randint(0, 40, (rows,), generator=g, device=DEV)
    ncand = (int(pos.min()) // 8)
    ids = torch.stack([torch.randperm(ncand, generator=g, device=DEV)[:512]
                       for _ in range(rows * 4)]).to(torch.int32).view(rows, 4, 512).contiguous()
    return q, k, v, ids, seq, pos.to(torch.int64)


@pytest.mark.parametrize("Hq,D", [(16, 128), (64, 192)])
def test_noalloc_equals_workspace_call_twice(Hq, D):
    for rows, seed in ((16, 3), (5, 4)):
        q, k, v, ids, seq, pos = _inputs(rows, Hq, D, 6000, seed)
        assert s5.step5_sparse_attn_workspace(rows, Hq, D) > 0
        scale = 1.0 / math.sqrt(D)
        out_ref = torch.full((rows, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse_ref = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device=DEV)
        s5.step5_sparse_attn(q, k, v, ids, seq, pos, scale, out_ref, lse_ref)
        out = torch.full_like(out_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        s5.step5_sparse_attn_noalloc(q, k, v, ids, seq, pos, scale, out, lse)
        torch.cuda.synchronize()
        print(f"[case] noalloc Hq={Hq} D={D} rows={rows}", flush=True)
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), (rows, "out")
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), (rows, "lse")
