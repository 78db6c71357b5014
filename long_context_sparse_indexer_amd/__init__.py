"""Step-5 sparse-indexer (DSA/CSA) hot path on AMD Instinct MI355X (gfx950).

A thin binding over libstep5.so, the C ABI declared in include/step5.h. The
functions carry the C names and only marshal arguments: they take torch
tensors for device memory, pass their pointers, strides and the current HIP
stream, and raise Step5Error on a non-zero status. Every step of the path runs
in the library's HIP kernels; there is no other implementation behind these
functions, and importing them without the built library raises.

Source of the method: TensorFold pull request #903, "Step-5-Preview on one
256 GB Mac" (indexer commit note), see include/step5.h.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

__all__ = [
    "Step5Error", "GEOM", "lib", "step5_status_str", "step5_index_summarize",
    "step5_index_append", "step5_index_score_topk", "step5_index_score_topk_workspace", "step5_sparse_attn",
    "step5_sparse_attn_workspace", "step5_sparse_attn_noalloc", "attn_geom", "STEP5_Q_E4M3", "STEP5_APPEND_ONE_PER_SEQ",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstep5.so")
STEP5_Q_E4M3 = 1
STEP5_APPEND_ONE_PER_SEQ = 1

IDX_HEADS, GROUPS, IDX_DIM, ROPE_DIM, REGION, TOPK = 16, 4, 64, 32, 8, 512
Q_HEADS, KV_HEADS, HEAD_DIM = 16, 4, 128


class Step5Geom(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("idx_heads", "groups", "idx_dim", "rope_dim", "region",
                                         "topk", "q_heads", "kv_heads", "head_dim")]


GEOM = Step5Geom(IDX_HEADS, GROUPS, IDX_DIM, ROPE_DIM, REGION, TOPK, Q_HEADS, KV_HEADS, HEAD_DIM)


class Step5ProjOut(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_row", C.c_int64)]


# outputs of the fused projection, in the order of the weight's rows
PROJ_PARTS = ("q", "k", "v", "index_q", "index_k", "index_z", "gate")


class Step5Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({step5_status_str(status)})")
        self.status = status


_lib = None


def lib():
    """The loaded libstep5.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python -m long_context_sparse_indexer_amd._build")
        L = C.CDLL(LIB_PATH)
        P, I64, I32, F, U32, SZ = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_uint32, C.c_size_t
        G = C.POINTER(Step5Geom)
        L.step5_status_str.restype = C.c_char_p
        L.step5_status_str.argtypes = [C.c_int]
        L.step5_index_summarize.restype = C.c_int
        L.step5_index_summarize.argtypes = [G, P, P, I64, I64, I64, I64, I64, P, P, F, P, I64, P,
                                            I64, I64, P]
        L.step5_index_append.restype = C.c_int
        L.step5_index_append.argtypes = [G, U32, P, P, I64, P, P, I32, P, P, I64, I64, I64, P, P, F, P,
                                         I64, P, I64, I64, P]
        L.step5_index_score_topk.restype = C.c_int
        L.step5_index_score_topk.argtypes = [G, U32, P, I64, P, F, P, I64, P, I64, P, P, I32, P,
                                             I64, I64, I64, P, P, P, SZ, P]
        L.step5_index_append_score_topk.restype = C.c_int
        L.step5_index_append_score_topk.argtypes = [G, U32, C.POINTER(Step5AppendIn), P, I64, P, F,
                                                    P, I64, P, I64, P, P, I32, P, I64, I64, I64, P,
                                                    P, P, SZ, P]
        L.step5_index_score_topk_workspace.restype = SZ
        L.step5_index_score_topk_workspace.argtypes = [G, I32, I64]
        L.step5_sparse_attn.restype = C.c_int
        L.step5_sparse_attn.argtypes = [G, P, I64, P, P, I64, I64, I64, I64, P, P, P, I32, F, P,
                                        P, P, SZ, P]
        L.step5_sparse_attn_noalloc.restype = C.c_int
        L.step5_sparse_attn_noalloc.argtypes = [G, P, I64, P, P, I64, I64, I64, I64, P, P, P, I32,
                                                F, P, P, P]
        L.step5_sparse_attn_workspace.restype = SZ
        L.step5_sparse_attn_workspace.argtypes = [G, I32]
        L.step5_qkv_index_project.restype = C.c_int
        L.step5_qkv_index_project.argtypes = [G, P, I64, I32, I32, P, I32, C.POINTER(Step5ProjOut), P]
        _lib = L
    return _lib


def step5_status_str(status: int) -> str:
    return lib().step5_status_str(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check(fn: str, status: int):
    if status != 0:
        raise Step5Error(fn, status)


def step5_index_summarize(k: torch.Tensor, z: torch.Tensor, t0: int, ln_w: torch.Tensor,
                          ln_b: torch.Tensor, ln_eps: float, rope: torch.Tensor,
                          summary: torch.Tensor, stream=None) -> None:
    """Summarise the regions completed in k/z (bf16 [B, T, 4, 64], positions t0..t0+T-1)
    into summary (e4m3 as uint8 [B, R_cap, 4, 64])."""
    _need(k.dtype == torch.bfloat16 and z.dtype == torch.bfloat16, "k, z must be bf16")
    _need(k.dim() == 4 and k.shape == z.shape and tuple(k.shape[2:]) == (GROUPS, IDX_DIM),
          "k, z must be [B, T, 4, 64]")
    _need(k.stride() == z.stride() and k.stride(3) == 1 and k.stride(2) == IDX_DIM,
          "k, z need contiguous (group, dim) and equal strides")
    summary = _u8(summary)
    _need(summary.dtype == torch.uint8 and summary.dim() == 4 and
          tuple(summary.shape[2:]) == (GROUPS, IDX_DIM) and summary.shape[0] == k.shape[0],
          "summary must be uint8 [B, R_cap, 4, 64]")
    _need(summary.stride(3) == 1 and summary.stride(2) == IDX_DIM and
          summary.stride(1) == GROUPS * IDX_DIM, "summary regions must be contiguous")
    _need(rope.dtype == torch.bfloat16 and rope.dim() == 2 and rope.shape[1] == ROPE_DIM and
          rope.is_contiguous(), "rope must be contiguous bf16 [rows, 32]")
    B, T = k.shape[0], k.shape[1]
    st = lib().step5_index_summarize(
        C.byref(GEOM), _ptr(k), _ptr(z), B, T, int(t0), k.stride(0), k.stride(1), _ptr(ln_w),
        _ptr(ln_b), float(ln_eps), _ptr(rope), rope.shape[0], _ptr(summary), summary.stride(0),
        summary.shape[1], _stream(stream))
    _check("step5_index_summarize", st)


def _append_checks(k_new, z_new, row_seq, row_pos, k_ring, z_ring, summary, rope):
    _need(k_new.dtype == torch.bfloat16 and z_new.dtype == torch.bfloat16, "k_new, z_new must be bf16")
    _need(k_new.dim() == 3 and k_new.shape == z_new.shape and
          tuple(k_new.shape[1:]) == (GROUPS, IDX_DIM), "k_new, z_new must be [rows, 4, 64]")
    _need(k_new.stride() == z_new.stride() and k_new.stride(2) == 1 and k_new.stride(1) == IDX_DIM,
          "k_new, z_new need contiguous (group, dim) and equal strides")
    _need(k_ring.dtype == torch.bfloat16 and z_ring.dtype == torch.bfloat16 and
          k_ring.dim() == 4 and k_ring.shape == z_ring.shape and
          tuple(k_ring.shape[2:]) == (GROUPS, IDX_DIM), "rings must be bf16 [B, slots, 4, 64]")
    _need(k_ring.stride() == z_ring.stride() and k_ring.stride(3) == 1 and
          k_ring.stride(2) == IDX_DIM and k_ring.stride(1) == GROUPS * IDX_DIM,
          "ring slots must be contiguous, both rings alike")
    summary = _u8(summary)
    _need(summary.dtype == torch.uint8 and summary.dim() == 4 and
          tuple(summary.shape[2:]) == (GROUPS, IDX_DIM) and summary.shape[0] == k_ring.shape[0],
          "summary must be uint8 [B, R_cap, 4, 64]")
    _need(summary.stride(3) == 1 and summary.stride(2) == IDX_DIM and
          summary.stride(1) == GROUPS * IDX_DIM, "summary regions must be contiguous")
    _need(rope.dtype == torch.bfloat16 and rope.dim() == 2 and rope.shape[1] == ROPE_DIM and
          rope.is_contiguous(), "rope must be contiguous bf16 [rows, 32]")
    _need(row_seq.dtype == torch.int32 and row_pos.dtype == torch.int64 and
          row_seq.is_contiguous() and row_pos.is_contiguous() and
          row_seq.numel() == k_new.shape[0] and row_pos.numel() == k_new.shape[0],
          "row_seq int32 [rows], row_pos int64 [rows], contiguous")
    return summary


def step5_index_append(k_new: torch.Tensor, z_new: torch.Tensor, row_seq: torch.Tensor,
                       row_pos: torch.Tensor, k_ring: torch.Tensor, z_ring: torch.Tensor,
                       ln_w: torch.Tensor, ln_b: torch.Tensor, ln_eps: float, rope: torch.Tensor,
                       summary: torch.Tensor, one_per_seq: bool = False, stream=None) -> None:
    """Write each row's new token (k_new, z_new: bf16 [rows, 4, 64]) to slot
    row_pos mod slots of its sequence's rings (k_ring, z_ring: bf16
    [B, slots, 4, 64]) and summarise the regions those tokens complete into
    summary (e4m3 as uint8 [B, R_cap, 4, 64]). one_per_seq: no two rows share a
    sequence (a decode step), which lets the call run as one launch."""
    summary = _append_checks(k_new, z_new, row_seq, row_pos, k_ring, z_ring, summary, rope)
    st = lib().step5_index_append(
        C.byref(GEOM), STEP5_APPEND_ONE_PER_SEQ if one_per_seq else 0, _ptr(k_new), _ptr(z_new),
        k_new.stride(0), _ptr(row_seq), _ptr(row_pos),
        k_new.shape[0], _ptr(k_ring), _ptr(z_ring), k_ring.shape[0], k_ring.shape[1],
        k_ring.stride(0), _ptr(ln_w), _ptr(ln_b), float(ln_eps), _ptr(rope), rope.shape[0],
        _ptr(summary), summary.stride(0), summary.shape[1], _stream(stream))
    _check("step5_index_append", st)


def step5_index_score_topk_workspace(rows: int, R_cap: int) -> int:
    return int(lib().step5_index_score_topk_workspace(C.byref(GEOM), int(rows), int(R_cap)))


def attn_geom(q_heads: int = Q_HEADS, head_dim: int = HEAD_DIM) -> Step5Geom:
    """The layer geometry with the given attention query heads (4, 8 or 16 per
    KV head) and head dim (128 or 192); the indexer part is fixed."""
    return Step5Geom(IDX_HEADS, GROUPS, IDX_DIM, ROPE_DIM, 8, TOPK, int(q_heads), KV_HEADS,
                     int(head_dim))


def step5_sparse_attn_workspace(rows: int, q_heads: int = Q_HEADS, head_dim: int = HEAD_DIM) -> int:
    return int(lib().step5_sparse_attn_workspace(C.byref(attn_geom(q_heads, head_dim)), int(rows)))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return workspace
    if workspace is None:
        # zero-filled: the attention workspace's arrival counters start at zero
        workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-workspace.data_ptr()) % 256
        workspace = workspace[off:off + nbytes]
    _need(workspace.numel() >= nbytes, f"workspace needs {nbytes} bytes")
    return workspace


def _score_checks(q, w_head, row_seq, row_pos, summary, sel_ids, sel_scores, q_norm_w, rope,
                  q_is_e4m3, workspace):
    q = _u8(q) if q_is_e4m3 else q
    rows = q.shape[0]
    _need(q.dim() == 3 and tuple(q.shape[1:]) == (IDX_HEADS, IDX_DIM) and q.stride(2) == 1 and
          q.stride(1) == IDX_DIM, "q must be [rows, 16, 64] with contiguous heads")
    _need(q.dtype == (torch.uint8 if q_is_e4m3 else torch.bfloat16), "q dtype")
    summary = _u8(summary)
    _need(summary.dtype == torch.uint8 and summary.dim() == 4 and summary.stride(1) == 256 and
          summary.stride(2) == 64 and summary.stride(3) == 1, "summary must be uint8 [B, R_cap, 4, 64]")
    _need(w_head.dtype == torch.float32 and w_head.shape[-1] == IDX_HEADS and w_head.stride(-1) == 1,
          "w_head must be fp32 [16] or [rows, 16]")
    w_stride = 0 if w_head.dim() == 1 else w_head.stride(0)
    _need(row_seq.dtype == torch.int32 and row_pos.dtype == torch.int64 and
          row_seq.numel() == rows and row_pos.numel() == rows, "row_seq int32 / row_pos int64 [rows]")
    _need(sel_ids.dtype == torch.int32 and tuple(sel_ids.shape) == (rows, GROUPS, TOPK) and
          sel_ids.is_contiguous(), "sel_ids must be int32 [rows, 4, 512]")
    if sel_scores is not None:
        _need(sel_scores.dtype == torch.float32 and sel_scores.shape == sel_ids.shape and
              sel_scores.is_contiguous(), "sel_scores must be fp32 [rows, 4, 512]")
    if not q_is_e4m3:
        _need(q_norm_w is not None and rope is not None, "q_norm_w and rope are needed")
    B, R_cap = summary.shape[0], summary.shape[1]
    nbytes = step5_index_score_topk_workspace(rows, R_cap)
    workspace = _workspace(nbytes, q.device, workspace)
    return q, rows, summary, w_stride, B, R_cap, nbytes, workspace


def step5_index_score_topk(q: torch.Tensor, w_head: torch.Tensor, row_seq: torch.Tensor,
                           row_pos: torch.Tensor, summary: torch.Tensor, sel_ids: torch.Tensor,
                           sel_scores: Optional[torch.Tensor] = None, *,
                           q_norm_w: Optional[torch.Tensor] = None, q_eps: float = 1e-6,
                           rope: Optional[torch.Tensor] = None, q_is_e4m3: bool = False,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Scores and top-512 per (row, group) into sel_ids (int32 [rows, 4, 512])."""
    q, rows, summary, w_stride, B, R_cap, nbytes, workspace = _score_checks(
        q, w_head, row_seq, row_pos, summary, sel_ids, sel_scores, q_norm_w, rope, q_is_e4m3,
        workspace)
    st = lib().step5_index_score_topk(
        C.byref(GEOM), STEP5_Q_E4M3 if q_is_e4m3 else 0, _ptr(q), q.stride(0), _ptr(q_norm_w),
        float(q_eps), _ptr(rope), rope.shape[0] if rope is not None else 0, _ptr(w_head), w_stride,
        _ptr(row_seq), _ptr(row_pos), rows, _ptr(summary), B, R_cap, summary.stride(0),
        _ptr(sel_ids), _ptr(sel_scores), _ptr(workspace), nbytes, _stream(stream))
    _check("step5_index_score_topk", st)


class Step5AppendIn(C.Structure):
    """The append half of step5_index_append_score_topk (step5_append_in)."""
    _fields_ = [("k_new", C.c_void_p), ("z_new", C.c_void_p), ("new_stride_row", C.c_int64),
                ("k_ring", C.c_void_p), ("z_ring", C.c_void_p), ("ring_slots", C.c_int64),
                ("ring_stride_b", C.c_int64), ("ln_w", C.c_void_p), ("ln_b", C.c_void_p),
                ("ln_eps", C.c_float)]


def step5_index_append_score_topk(k_new: torch.Tensor, z_new: torch.Tensor, k_ring: torch.Tensor,
                                  z_ring: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                                  ln_eps: float, q: torch.Tensor, w_head: torch.Tensor,
                                  row_seq: torch.Tensor, row_pos: torch.Tensor,
                                  summary: torch.Tensor, sel_ids: torch.Tensor,
                                  sel_scores: Optional[torch.Tensor] = None, *,
                                  rope: torch.Tensor, q_norm_w: Optional[torch.Tensor] = None,
                                  q_eps: float = 1e-6, q_is_e4m3: bool = False,
                                  workspace: Optional[torch.Tensor] = None, stream=None,
                                  check_distinct: bool = False) -> None:
    """step5_index_append (rows of distinct sequences) and
    step5_index_score_topk of the same rows in one call: the appends run in
    extra workgroups of the selection's launch. The rows must not share a
    sequence: the library cannot check it (device values); check_distinct
    checks it here first (a host synchronisation, so not inside a HIP graph
    capture) and raises ValueError when two rows name one sequence."""
    if check_distinct:
        _need(row_seq.dim() == 1 and int(torch.unique(row_seq).numel()) == row_seq.numel(),
              "step5_index_append_score_topk: two rows share a sequence")
    summary = _append_checks(k_new, z_new, row_seq, row_pos, k_ring, z_ring, summary, rope)
    q, rows, summary, w_stride, B, R_cap, nbytes, workspace = _score_checks(
        q, w_head, row_seq, row_pos, summary, sel_ids, sel_scores, q_norm_w, rope, q_is_e4m3,
        workspace)
    _need(k_new.shape[0] == rows, "k_new and q must have the same rows")
    ap = Step5AppendIn(_ptr(k_new), _ptr(z_new), k_new.stride(0), _ptr(k_ring), _ptr(z_ring),
                       k_ring.shape[1], k_ring.stride(0), _ptr(ln_w), _ptr(ln_b), float(ln_eps))
    st = lib().step5_index_append_score_topk(
        C.byref(GEOM), STEP5_Q_E4M3 if q_is_e4m3 else 0, C.byref(ap), _ptr(q), q.stride(0),
        _ptr(q_norm_w), float(q_eps), _ptr(rope), rope.shape[0], _ptr(w_head), w_stride,
        _ptr(row_seq), _ptr(row_pos), rows, _ptr(summary), B, R_cap, summary.stride(0),
        _ptr(sel_ids), _ptr(sel_scores), _ptr(workspace), nbytes, _stream(stream))
    _check("step5_index_append_score_topk", st)


def _attn_checks(q, k_cache, v_cache, sel_ids, row_seq, row_pos, out, out_lse):
    rows = q.shape[0]
    _need(q.dtype == torch.bfloat16 and q.dim() == 3 and q.stride(2) == 1 and
          q.stride(1) == q.shape[2], "q must be bf16 [rows, Hq, D] with contiguous heads")
    Hq, D = q.shape[1], q.shape[2]
    _need(k_cache.dtype == torch.bfloat16 and v_cache.dtype == torch.bfloat16 and
          k_cache.shape == v_cache.shape and k_cache.stride() == v_cache.stride() and
          k_cache.dim() == 4 and tuple(k_cache.shape[2:]) == (KV_HEADS, D) and
          k_cache.stride(3) == 1 and k_cache.stride(2) == D,
          "k_cache, v_cache must be bf16 [B, T, 4, D] with equal strides")
    _need(sel_ids.dtype == torch.int32 and tuple(sel_ids.shape) == (rows, GROUPS, TOPK) and
          sel_ids.is_contiguous(), "sel_ids must be int32 [rows, 4, 512]")
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (rows, Hq, D) and
          out.is_contiguous(), "out must be contiguous bf16 [rows, Hq, D]")
    if out_lse is not None:
        _need(out_lse.dtype == torch.float32 and tuple(out_lse.shape) == (rows, Hq) and
              out_lse.is_contiguous(), "out_lse must be fp32 [rows, Hq]")
    _need(row_seq.dtype == torch.int32 and row_pos.dtype == torch.int64, "row_seq int32, row_pos int64")
    return rows, attn_geom(Hq, D)


def step5_sparse_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      sel_ids: torch.Tensor, row_seq: torch.Tensor, row_pos: torch.Tensor,
                      softmax_scale: float, out: torch.Tensor,
                      out_lse: Optional[torch.Tensor] = None, *,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Attention over selected regions plus the own region into out (bf16 [rows, Hq, D]).
    The geometry comes from q: Hq query heads (16, 32 or 64: 4, 8 or 16 per KV
    head) of D = 128 or 192 dims; k_cache, v_cache bf16 [B, T, 4, D]."""
    rows, geom = _attn_checks(q, k_cache, v_cache, sel_ids, row_seq, row_pos, out, out_lse)
    nbytes = int(lib().step5_sparse_attn_workspace(C.byref(geom), int(rows)))
    workspace = _workspace(nbytes, q.device, workspace)
    st = lib().step5_sparse_attn(
        C.byref(geom), _ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        k_cache.stride(0), k_cache.stride(1), k_cache.shape[1], _ptr(sel_ids), _ptr(row_seq),
        _ptr(row_pos), rows, float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
        nbytes, _stream(stream))
    _check("step5_sparse_attn", st)


def step5_sparse_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              sel_ids: torch.Tensor, row_seq: torch.Tensor, row_pos: torch.Tensor,
                              softmax_scale: float, out: torch.Tensor,
                              out_lse: Optional[torch.Tensor] = None, *, stream=None) -> None:
    """step5_sparse_attn without a workspace: the library's static device
    scratch holds the split states (no allocation, for graph capture and
    serving loops). Calls that overlap on one GPU share that scratch."""
    rows, geom = _attn_checks(q, k_cache, v_cache, sel_ids, row_seq, row_pos, out, out_lse)
    st = lib().step5_sparse_attn_noalloc(
        C.byref(geom), _ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        k_cache.stride(0), k_cache.stride(1), k_cache.shape[1], _ptr(sel_ids), _ptr(row_seq),
        _ptr(row_pos), rows, float(softmax_scale), _ptr(out), _ptr(out_lse), _stream(stream))
    _check("step5_sparse_attn_noalloc", st)


def proj_widths(gate_size: int = Q_HEADS, q_heads: int = Q_HEADS, head_dim: int = HEAD_DIM):
    """Columns of each output of the fused projection (PROJ_PARTS order)."""
    return (q_heads * head_dim, KV_HEADS * head_dim, KV_HEADS * head_dim, IDX_HEADS * IDX_DIM,
            GROUPS * IDX_DIM, GROUPS * IDX_DIM, gate_size)


def step5_qkv_index_project(hidden: torch.Tensor, weight: torch.Tensor, outs, *,
                            gate_size: int = Q_HEADS, q_heads: int = Q_HEADS,
                            head_dim: int = HEAD_DIM, stream=None) -> None:
    """outs[part] = the part's columns of hidden (bf16 [rows, H]) @ weight^T
    (weight bf16 [N, H], rows in PROJ_PARTS order); outs: a sequence of 7
    bf16 tensors [rows, width] (PROJ_PARTS order, rows of stride >= width)."""
    _need(hidden.dtype == torch.bfloat16 and hidden.dim() == 2 and hidden.stride(1) == 1,
          "hidden must be bf16 [rows, H] with contiguous rows")
    rows, H = hidden.shape
    widths = proj_widths(gate_size, q_heads, head_dim)
    _need(weight.dtype == torch.bfloat16 and tuple(weight.shape) == (sum(widths), H) and
          weight.is_contiguous(), f"weight must be contiguous bf16 [{sum(widths)}, {H}]")
    _need(len(outs) == len(PROJ_PARTS), "outs must hold 7 tensors")
    arr = (Step5ProjOut * len(PROJ_PARTS))()
    for i, (t, wdt) in enumerate(zip(outs, widths)):
        _need(t.dtype == torch.bfloat16 and t.dim() == 2 and tuple(t.shape) == (rows, wdt) and
              t.stride(1) == 1, f"{PROJ_PARTS[i]} must be bf16 [{rows}, {wdt}] with contiguous rows")
        arr[i].ptr = t.data_ptr() if wdt else None
        arr[i].stride_row = t.stride(0) if rows > 1 else max(wdt, 8)
    geom = attn_geom(q_heads, head_dim)
    st = lib().step5_qkv_index_project(C.byref(geom), _ptr(hidden), hidden.stride(0) if rows > 1 else H,
                                       rows, H, _ptr(weight), gate_size, arr, _stream(stream))
    _check("step5_qkv_index_project", st)
