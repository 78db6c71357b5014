"""GPU parity of the incremental indexer-cache update (step5_index_append):
tokens streamed into the k/z rings one at a time or in prompt-sized chunks
leave exactly the e4m3 summaries the oracle's batch summary writes from the
contiguous k and z, the rings hold each slot's latest token, and nothing
else is written.

Source: TensorFold pull request #903 "Step-5-Preview on one 256 GB Mac"
(prompt-path commit note: the indexer's k and z live in rings holding one
prompt chunk more than a chunk; indexer commit note: every completed region
is summarised).
"""
import numpy as np
import pytest
import torch

import workloads as W
import parity as P
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _stream_gpu(d, slots, chunks, R_cap, sentinel=0x55, one_per_seq=False):
    """Feed every sequence's tokens through the GPU append, the same chunk of
    positions for all sequences in one call (rows interleaved by sequence)."""
    k, z = d["k_idx"].to(DEV), d["z_idx"].to(DEV)
    B, T = k.shape[:2]
    k_ring = torch.zeros((B, slots, 4, 64), dtype=torch.bfloat16, device=DEV)
    z_ring = torch.zeros_like(k_ring)
    S = torch.full((B, R_cap, 4, 64), sentinel, dtype=torch.uint8, device=DEV)
    lnw, lnb, rope = d["ln_w"].to(DEV), d["ln_b"].to(DEV), d["rope"].to(DEV)
    t = 0
    for n in chunks:
        pos = torch.arange(t, t + n, dtype=torch.int64, device=DEV).repeat(B)
        seq = torch.arange(B, dtype=torch.int32, device=DEV).repeat_interleave(n)
        kn = k[:, t:t + n].reshape(B * n, 4, 64)
        zn = z[:, t:t + n].reshape(B * n, 4, 64)
        s5 = P.s5
        s5.step5_index_append(kn, zn, seq, pos, k_ring, z_ring, lnw, lnb, P.EPS, rope, S,
                              one_per_seq=one_per_seq)
        t += n
    assert t == T
    torch.cuda.synchronize()
    return k_ring, z_ring, S


def _oracle_batch(d, R_cap, sentinel=0x55):
    base = np.full((d["k_idx"].shape[0], R_cap, 4, 64), sentinel, np.uint8)
    return orc.summarize(P.host16(d["k_idx"]), P.host16(d["z_idx"]), 0, d["ln_w"].numpy(),
                         d["ln_b"].numpy(), P.EPS, P.host16(d["rope"]), R_cap=R_cap, summary=base)


@pytest.mark.parametrize("chunks,one", [([1] * 101, False), ([1] * 101, True),
                                        ([5, 11, 16, 17, 1, 7, 13, 8, 17, 6], False)])
def test_append_stream_equals_batch_summary(chunks, one):
    """3 sequences of 101 tokens through a 24-slot ring: one token per call
    (decode; also as the one-launch path, each sequence once per call) and
    chunks of up to 17 = 24 - 8 + 1 tokens (prompt)."""
    d = W.make_case(W.WORKLOADS["decode8_ctx3000"], 17, "cpu", cache_tokens=101, rows=3, batch=3,
                    with_kv=False)
    P.say(f"[case] append stream chunks={chunks[:4]}... one_per_seq={one} B=3 T=101 slots=24")
    R_cap = 14
    k_ring, z_ring, S = _stream_gpu(d, 24, chunks, R_cap, one_per_seq=one)
    O = _oracle_batch(d, R_cap)
    got = S.cpu().numpy()
    assert np.array_equal(got, O)
    assert np.all(got[:, 12:] == 0x55)           # tokens 96..100: region 12 still open
    kh, zh = P.host16(k_ring), P.host16(z_ring)
    k16, z16 = P.host16(d["k_idx"]), P.host16(d["z_idx"])
    for i in range(24):
        last = max(p for p in range(101) if p % 24 == i)
        assert np.array_equal(kh[:, i], k16[:, last]) and np.array_equal(zh[:, i], z16[:, last])


def test_append_skips_invalid_rows_and_open_regions():
    d = W.make_case(W.WORKLOADS["decode8_ctx3000"], 41, "cpu", cache_tokens=16, rows=2, batch=2,
                    with_kv=False)
    P.say("[case] append invalid rows")
    k, z = d["k_idx"].to(DEV), d["z_idx"].to(DEV)
    k_ring = torch.zeros((2, 8, 4, 64), dtype=torch.bfloat16, device=DEV)
    z_ring = torch.zeros_like(k_ring)
    S = torch.full((2, 1, 4, 64), 0x55, dtype=torch.uint8, device=DEV)
    # sequence 2 and -1 do not exist; position 8 lies in region 1 >= R_cap;
    # position 5 is valid but completes nothing
    seq = torch.tensor([2, -1, 0, 1], dtype=torch.int32, device=DEV)
    pos = torch.tensor([7, 7, 8, 5], dtype=torch.int64, device=DEV)
    P.s5.step5_index_append(k[0, :4].contiguous(), z[0, :4].contiguous(), seq, pos, k_ring,
                            z_ring, d["ln_w"].to(DEV), d["ln_b"].to(DEV), P.EPS,
                            d["rope"].to(DEV), S)
    torch.cuda.synchronize()
    kh = P.host16(k_ring)
    assert np.all(kh[0] == 0) and np.all(np.delete(kh[1], 5, axis=0) == 0)
    assert np.array_equal(kh[1, 5], P.host16(d["k_idx"])[0, 3])
    assert np.all(S.cpu().numpy() == 0x55)


@pytest.mark.parametrize("one", [False, True])
def test_append_full_size_decode16_ctx128k(one):
    """The decode16_ctx128k step's cache update: 16 rows at position 131,071
    complete region 16,383 from a 520-slot ring (one 512-token chunk plus a
    region) holding the other 7 tokens; checked against the oracle's batch
    summary of that region."""
    d = W.make_case(W.WORKLOADS["decode16_ctx128k"], 23, DEV, with_kv=False)
    P.say(f"[case] append decode16_ctx128k full size one_per_seq={one}")
    k, z = d["k_idx"], d["z_idx"]
    B, T = k.shape[:2]
    slots, R_cap = 520, T // 8
    p = T - 1
    k_ring = torch.zeros((B, slots, 4, 64), dtype=torch.bfloat16, device=DEV)
    z_ring = torch.zeros_like(k_ring)
    for t in range(p - 7, p):                      # the region's earlier tokens
        k_ring[:, t % slots] = k[:, t]
        z_ring[:, t % slots] = z[:, t]
    S = torch.full((B, R_cap, 4, 64), 0xA5, dtype=torch.uint8, device=DEV)
    seq = torch.arange(B, dtype=torch.int32, device=DEV)
    pos = torch.full((B,), p, dtype=torch.int64, device=DEV)
    P.s5.step5_index_append(k[:, p].contiguous(), z[:, p].contiguous(), seq, pos, k_ring, z_ring,
                            d["ln_w"], d["ln_b"], P.EPS, d["rope"], S, one_per_seq=one)
    torch.cuda.synchronize()
    got = S.cpu().numpy()
    assert np.all(got[:, :R_cap - 1] == 0xA5)
    O = orc.summarize(P.host16(k[:, p - 7:p + 1]), P.host16(z[:, p - 7:p + 1]), p - 7,
                      d["ln_w"].cpu().numpy(), d["ln_b"].cpu().numpy(), P.EPS,
                      P.host16(d["rope"]), R_cap=R_cap)
    assert np.array_equal(got[:, R_cap - 1], O[:, R_cap - 1])
    assert np.array_equal(P.host16(k_ring[:, p % slots]), P.host16(k[:, p]))
    assert np.array_equal(P.host16(z_ring[:, p % slots]), P.host16(z[:, p]))
