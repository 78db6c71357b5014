"""Seeded synthetic inputs for the Step-5 sparse-indexer path.

This module only draws inputs. It holds none of the path's arithmetic, and it
is the one piece that the GPU library's callers and the CPU oracle's callers
share: both receive the same bytes.

Five workloads, named by what they are:

  decode1_ctx6000     one decode row at position 5,999 of a 6,000-token cache
                      (750 completed regions, so the top-512 cut is exercised)
  decode8_ctx3000     8 sequences of 3,000 tokens, one decode row each at
                      position 2,999 (374 candidates: every region selected;
                      the output equals dense causal attention); z scaled by 2
  prefill2048_ctx32k  a chunk of 2,048 query rows at positions 30,720..32,767
                      of one 32,768-token sequence (4,096 regions); w ~ U(0,1)
  decode16_ctx128k    16 sequences of 131,072 tokens, one decode row each at
                      position 131,071; activations Student-t (nu = 3) scaled
                      to unit variance
  decode1_ctx1m       one decode row at position 1,048,575 of a 1,048,576-token
                      cache; prepared q and the region summaries are drawn
                      directly as e4m3 from {+-1/4, +-1/2, +-1, +-2} and
                      w_h = (h + 1) / 16, so that scores tie exactly and often;
                      plus a summary pass over a fresh 65,536-token span

Layer shapes (the Step-5 full-attention layer): indexer 16 heads x 64 dims in
4 KV groups, NEOX rotation on dims 0..31 (base 10,000), regions of 8 tokens,
top 512; main attention 16 q heads over 4 KV heads of 128 dims, bf16.

Positions are 0-based and a cache of T tokens holds positions 0..T-1, so the
row "at position 6,000" of a 6,000-token cache is position 5,999.

Parameter draws the pages do not give: q-norm weight w ~ U(-0.5, 0.5) (the
norm scales by 1 + w), LayerNorm weight ~ U(0.5, 1.5), bias ~ U(-0.5, 0.5),
head weights w_h ~ U(0, 1); all fp32.

Every tensor comes from torch's generator seeded with the given seed, on the
device asked for (a CPU generator for CPU tensors, the device's own generator
for GPU tensors). Generating on the GPU is how the full-size workloads are
made quickly; tests copy the GPU tensors' bytes back to the host for the
oracle, so both sides still read identical inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

IDX_HEADS = 16
GROUPS = 4
IDX_DIM = 64
ROT_DIM = 32
REGION = 8
TOPK = 512
Q_HEADS = 16
KV_HEADS = 4
HEAD_DIM = 128
ROPE_BASE = 10000.0
NORM_EPS = 1e-6

# e4m3 (OCP) codes of +1/4, +1/2, +1, +2 and their negatives
TIE_CODES = (0x28, 0x30, 0x38, 0x40, 0xA8, 0xB0, 0xB8, 0xC0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int              # sequences in the caches
    cache_tokens: int       # tokens per sequence held in the caches
    rows: int               # query rows
    dist: str               # "normal" | "student3"
    z_scale: float = 1.0
    w_dist: str = "uniform01"   # head-weight draw: "uniform01" | "ramp16"
    tie_heavy: bool = False     # q8 and summaries drawn directly from TIE_CODES
    prefill_chunk: int = 0      # rows form one chunk of one sequence
    fresh_tokens: int = 0       # extra summary pass over a fresh span

    @property
    def regions(self) -> int:
        return self.cache_tokens // REGION

    def row_layout(self):
        """(row_seq, row_pos) as python lists."""
        if self.prefill_chunk:
            p0 = self.cache_tokens - self.rows
            return [0] * self.rows, list(range(p0, self.cache_tokens))
        return list(range(self.rows)), [self.cache_tokens - 1] * self.rows


WORKLOADS = {
    "decode1_ctx6000": Workload("decode1_ctx6000", 1, 6000, 1, "normal"),
    "decode8_ctx3000": Workload("decode8_ctx3000", 8, 3000, 8, "normal", z_scale=2.0),
    "prefill2048_ctx32k": Workload("prefill2048_ctx32k", 1, 32768, 2048, "normal",
                                   prefill_chunk=2048),
    "decode16_ctx128k": Workload("decode16_ctx128k", 16, 131072, 16, "student3"),
    "decode1_ctx1m": Workload("decode1_ctx1m", 1, 1048576, 1, "normal", w_dist="ramp16",
                              tie_heavy=True, fresh_tokens=65536),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw(shape, dist: str, g: torch.Generator, device) -> torch.Tensor:
    """fp32 draws of unit variance."""
    if dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if dist == "student3":
        # t with 3 degrees of freedom is N0 / sqrt(chi2_3 / 3) with chi2_3 the sum
        # of three squared normals; its variance is 3, so dividing by sqrt(3)
        # gives N0 / sqrt(N1^2 + N2^2 + N3^2).
        n = torch.randn((4,) + tuple(shape), generator=g, device=device, dtype=torch.float32)
        return n[0] / torch.sqrt(n[1] ** 2 + n[2] ** 2 + n[3] ** 2)
    raise ValueError(dist)


def _bf16(shape, dist, g, device, scale=1.0, chunk_elems=1 << 26) -> torch.Tensor:
    """bf16 draws, made in slices along dim 0 to bound fp32 scratch memory."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    per0 = max(1, math.prod(shape[1:]))
    step = max(1, chunk_elems // per0)
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        x = _draw((e - s,) + tuple(shape[1:]), dist, g, device)
        if scale != 1.0:
            x = x * scale
        out[s:e] = x.to(torch.bfloat16)
    return out


def _bf16_flat(n_tok, inner, dist, g, device, scale=1.0) -> torch.Tensor:
    return _bf16((n_tok,) + tuple(inner), dist, g, device, scale)


def rope_table(n_pos: int, device="cpu") -> torch.Tensor:
    """bf16 [n_pos, 32]: cos of the 16 NEOX frequencies, then their sin.

    inv_freq_i = base^(-2i/32) in fp32, angle = fp32(position) * inv_freq_i in
    fp32, cos/sin in fp32, then rounded to bf16: the usual fp32 recipe, kept
    in bf16 because the rotation reads bf16 cos/sin.
    """
    inv = 1.0 / (ROPE_BASE ** (torch.arange(0, ROT_DIM, 2, dtype=torch.float32) / ROT_DIM))
    pos = torch.arange(n_pos, dtype=torch.float32)
    ang = pos[:, None] * inv[None, :]
    tab = torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.bfloat16)
    return tab.to(device)


def _tie_codes(shape, g, device) -> torch.Tensor:
    idx = torch.randint(0, len(TIE_CODES), shape, generator=g, device=device)
    codes = torch.tensor(TIE_CODES, dtype=torch.uint8, device=device)
    return codes[idx]


def make_case(wl: Workload, seed: int, device="cpu", *, cache_tokens: Optional[int] = None,
              rows: Optional[int] = None, batch: Optional[int] = None,
              with_kv: bool = True, with_indexer_kz: bool = True) -> dict:
    """All inputs of one workload (optionally shrunk along tokens/rows/batch).

    Returns a dict of tensors on `device`:
      q_idx   bf16 [rows, 16, 64]     indexer q before prep (absent if tie_heavy)
      q8      uint8 [rows, 16, 64]    prepared e4m3 q (tie_heavy only)
      k_idx, z_idx  bf16 [B, T, 4, 64]  indexer k and z of the cache (absent if tie_heavy)
      summary uint8 [B, T/8, 4, 64]   e4m3 summaries (tie_heavy only)
      q_norm_w, ln_w, ln_b fp32 [64]; w_head fp32 [16]
      rope    bf16 [T, 32]
      q       bf16 [rows, 16, 128]    main-attention q (after its own rotation)
      k_cache, v_cache bf16 [B, T, 4, 128]
      row_seq int32 [rows], row_pos int64 [rows]
      fresh_k, fresh_z bf16 [1, F, 4, 64] and fresh_rope (when fresh_tokens)
    """
    T = cache_tokens or wl.cache_tokens
    R = rows or wl.rows
    B = batch or wl.batch
    if wl.prefill_chunk:
        R = min(R, T)
        row_seq = [0] * R
        row_pos = list(range(T - R, T))
    else:
        B = min(B, R) if batch is None else B
        row_seq = [i % B for i in range(R)]
        row_pos = [T - 1] * R
    g = _gen(seed, device)
    d = {"workload": wl.name, "batch": B, "cache_tokens": T, "rows": R}
    d["row_seq"] = torch.tensor(row_seq, dtype=torch.int32, device=device)
    d["row_pos"] = torch.tensor(row_pos, dtype=torch.int64, device=device)
    d["q_norm_w"] = torch.rand(IDX_DIM, generator=g, device=device) - 0.5
    d["ln_w"] = torch.rand(IDX_DIM, generator=g, device=device) + 0.5
    d["ln_b"] = torch.rand(IDX_DIM, generator=g, device=device) - 0.5
    if wl.w_dist == "ramp16":
        d["w_head"] = torch.arange(1, IDX_HEADS + 1, dtype=torch.float32, device=device) / 16.0
    else:
        d["w_head"] = torch.rand(IDX_HEADS, generator=g, device=device)
    if wl.tie_heavy:
        d["q8"] = _tie_codes((R, IDX_HEADS, IDX_DIM), g, device)
        d["summary"] = _tie_codes((B, T // REGION, GROUPS, IDX_DIM), g, device)
    else:
        d["q_idx"] = _bf16((R, IDX_HEADS, IDX_DIM), wl.dist, g, device)
        if with_indexer_kz:
            d["k_idx"] = _bf16((B, T, GROUPS, IDX_DIM), wl.dist, g, device)
            d["z_idx"] = _bf16((B, T, GROUPS, IDX_DIM), wl.dist, g, device, scale=wl.z_scale)
    d["q"] = _bf16((R, Q_HEADS, HEAD_DIM), wl.dist, g, device)
    if with_kv:
        d["k_cache"] = _bf16((B, T, KV_HEADS, HEAD_DIM), wl.dist, g, device)
        d["v_cache"] = _bf16((B, T, KV_HEADS, HEAD_DIM), wl.dist, g, device)
    n_rope = max(T, wl.fresh_tokens)
    d["rope"] = rope_table(n_rope, device)
    if wl.fresh_tokens:
        F = wl.fresh_tokens
        d["fresh_k"] = _bf16((1, F, GROUPS, IDX_DIM), "normal", g, device)
        d["fresh_z"] = _bf16((1, F, GROUPS, IDX_DIM), "normal", g, device)
    return d


def bits16(t: torch.Tensor):
    """Raw bits of a bf16 tensor as a numpy uint16 array (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def bits8(t: torch.Tensor):
    return t.detach().contiguous().cpu().numpy().view("uint8")
