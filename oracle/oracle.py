"""ctypes wrapper over the CPU oracle (libstep5_oracle.so).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
CPU-baseline leg. The GPU library never imports it.

All arrays are numpy, C-contiguous: bf16 as uint16 bit patterns, e4m3 as
uint8 codes.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("STEP5_ORACLE_LIB") or os.path.join(HERE, "libstep5_oracle.so")

IDX_DIM = 64
REGION = 8

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433
            _b.build()
        L = C.CDLL(LIB_PATH)
        P, I64, I32, F, D = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_double
        L.o_exp.restype = F
        L.o_exp.argtypes = [F]
        L.o_sum64.restype = F
        L.o_sum64.argtypes = [P]
        L.o_f32_to_bf16.restype = C.c_uint16
        L.o_f32_to_bf16.argtypes = [F]
        L.o_bf16_to_e4m3.restype = C.c_uint8
        L.o_bf16_to_e4m3.argtypes = [C.c_uint16]
        L.o_e4m3_to_f64.restype = D
        L.o_e4m3_to_f64.argtypes = [C.c_uint8]
        L.o_f32_to_bf16_n.argtypes = [P, P, I64]
        L.o_bf16_to_e4m3_n.argtypes = [P, P, I64]
        L.o_exp_n.argtypes = [P, P, I64, C.c_int]
        L.o_exp_bits_range.argtypes = [C.c_uint32, I64, P, C.c_int]
        L.o_k_prep_n.argtypes = [P, I64, P, P, F, P, P, P]
        L.o_q_prep_head.argtypes = [P, P, F, P, P]
        L.o_q_prep.restype = C.c_int
        L.o_q_prep.argtypes = [P, I64, I32, I64, P, F, P, I64, P, P, C.c_int]
        L.o_summarize.restype = C.c_int
        L.o_summarize.argtypes = [P, P, I64, I64, I64, I32, I64, I64, P, P, F, P, I64, P, I64, I64,
                                  P, C.c_int]
        L.o_score.restype = C.c_int
        L.o_score.argtypes = [P, I32, I32, P, I64, P, P, I64, P, I64, I64, I64, P, C.c_int]
        L.o_select.restype = C.c_int
        L.o_select.argtypes = [P, P, I64, I32, I64, I32, P, P, C.c_int]
        L.o_project.restype = C.c_int
        L.o_project.argtypes = [P, I64, I64, P, I64, P, C.c_int]
        L.o_attend.restype = C.c_int
        L.o_attend.argtypes = [P, I64, I32, I32, I32, P, P, I64, I64, I64, P, I32, P, P, I64, D,
                               P, P, C.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return int(os.environ.get("STEP5_ORACLE_THREADS", os.cpu_count() or 1))


# ---- formats and helpers ---------------------------------------------------

def f32_to_bf16(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().o_f32_to_bf16_n(_p(x), _p(y), x.size)
    return y


def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def bf16_to_e4m3(h) -> np.ndarray:
    h = _c(h, np.uint16)
    y = np.empty(h.shape, np.uint8)
    lib().o_bf16_to_e4m3_n(_p(h), _p(y), h.size)
    return y


def e4m3_to_f64(c) -> np.ndarray:
    table = np.array([lib().o_e4m3_to_f64(i) for i in range(256)], dtype=np.float64)
    return table[np.asarray(c, dtype=np.uint8)]


def exp(x, nthreads=None) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.float32)
    lib().o_exp_n(_p(x), _p(y), x.size, nthreads or default_threads())
    return y


def exp_bits_range(start: int, n: int, nthreads=None) -> np.ndarray:
    """exp of the n fp32 inputs with bit patterns start, start + 1, ..."""
    assert 0 <= start and start + n <= 1 << 32
    y = np.empty(n, np.float32)
    lib().o_exp_bits_range(start, n, _p(y), nthreads or default_threads())
    return y


def sum64(x) -> float:
    x = _c(x, np.float32)
    assert x.size == 64
    return float(lib().o_sum64(_p(x)))


def k_prep(x16, ln_w, ln_b, eps, rope, pos) -> np.ndarray:
    """Prepared k (fp32 values of bf16) for vectors x16 [n, 64] at positions pos [n]."""
    x16 = _c(x16, np.uint16).reshape(-1, IDX_DIM)
    pos = _c(pos, np.int64).reshape(-1)
    out = np.empty(x16.shape, np.float32)
    lib().o_k_prep_n(_p(x16), x16.shape[0], _p(_c(ln_w, np.float32)), _p(_c(ln_b, np.float32)),
                     float(eps), _p(_c(rope, np.uint16)), _p(pos), _p(out))
    return out


# ---- the path's steps ------------------------------------------------------

def q_prep(q16, w, eps, rope, row_pos, nthreads=None) -> np.ndarray:
    """q16: uint16 [rows, H, 64] -> e4m3 [rows, H, 64]."""
    q16 = _c(q16, np.uint16)
    rows, H, D = q16.shape
    assert D == IDX_DIM
    rope = _c(rope, np.uint16)
    out = np.empty(q16.shape, np.uint8)
    rc = lib().o_q_prep(_p(q16), rows, H, H * D, _p(_c(w, np.float32)), float(eps), _p(rope),
                        rope.shape[0], _p(_c(row_pos, np.int64)), _p(out),
                        nthreads or default_threads())
    if rc:
        raise ValueError("oracle q_prep rejected its arguments")
    return out


def summarize(k16, z16, t0, ln_w, ln_b, eps, rope, R_cap=None, summary=None, shadow=False,
              nthreads=None):
    """k16, z16: uint16 [B, T, G, 64] at absolute positions t0..t0+T-1.

    Returns the e4m3 summary [B, R_cap, G, 64] (regions outside the span are
    left as they were in `summary`, zero if it is None), and the fp64 shadow
    of the softmax means when asked for.
    """
    k16 = _c(k16, np.uint16)
    z16 = _c(z16, np.uint16)
    B, T, G, D = k16.shape
    assert D == IDX_DIM and z16.shape == k16.shape
    if R_cap is None:
        R_cap = (t0 + T) // REGION
    if summary is None:
        summary = np.zeros((B, R_cap, G, IDX_DIM), np.uint8)
    assert summary.shape == (B, R_cap, G, IDX_DIM) and summary.flags["C_CONTIGUOUS"]
    sh = np.full((B, R_cap, G, IDX_DIM), np.nan) if shadow else None
    rope = _c(rope, np.uint16)
    rc = lib().o_summarize(_p(k16), _p(z16), B, T, t0, G, T * G * D, G * D,
                           _p(_c(ln_w, np.float32)), _p(_c(ln_b, np.float32)), float(eps),
                           _p(rope), rope.shape[0], _p(summary), R_cap * G * D, R_cap,
                           _p(sh) if shadow else None, nthreads or default_threads())
    if rc:
        raise ValueError("oracle summarize rejected its arguments")
    return (summary, sh) if shadow else summary


def append(k_new, z_new, row_seq, row_pos, k_ring, z_ring, ln_w, ln_b, eps, rope, summary):
    """Indexer cache update for one new token per row, in place.

    TensorFold #903 ("Step-5-Preview on one 256 GB Mac"): the prompt-path
    commit note keeps the indexer's k and z in rings that hold one prompt
    chunk more than it needs; the indexer commit note summarises every
    completed 8-token region. Written out:
      1. row r's raw k and z go to slot row_pos[r] mod slots of sequence
         row_seq[r] (all rows first);
      2. every row whose token ends a region (p mod 8 == 7) has that region,
         p // 8, summarised from the ring slots of its tokens p-7 .. p, as the
         batch summary does it from contiguous k and z.
    k_new, z_new: uint16 [rows, G, 64]; k_ring, z_ring: uint16 [B, slots, G,
    64]; summary: uint8 [B, R_cap, G, 64]. Rows whose sequence is outside
    0..B-1, or whose position is negative, past the rope table or in a region
    >= R_cap, are skipped.
    """
    B, slots = k_ring.shape[:2]
    assert slots % REGION == 0 and slots >= REGION and z_ring.shape == k_ring.shape
    assert k_ring.flags["C_CONTIGUOUS"] and z_ring.flags["C_CONTIGUOUS"]
    R_cap = summary.shape[1]
    done = []
    for r in range(len(row_seq)):
        s, p = int(row_seq[r]), int(row_pos[r])
        if not (0 <= s < B and 0 <= p < rope.shape[0] and p // REGION < R_cap):
            continue
        k_ring[s, p % slots] = k_new[r]
        z_ring[s, p % slots] = z_new[r]
        done.append((s, p))
    for s, p in done:
        if p % REGION != REGION - 1:
            continue
        a = p - (REGION - 1)
        sl = a % slots
        summarize(k_ring[s:s + 1, sl:sl + REGION], z_ring[s:s + 1, sl:sl + REGION], a, ln_w,
                  ln_b, eps, rope, R_cap=R_cap, summary=summary[s:s + 1])
    return k_ring, z_ring, summary


def score(q8, w_head, row_seq, row_pos, summary, nthreads=None) -> np.ndarray:
    """q8 [rows, H, 64] e4m3; w_head [H] or [rows, H]; summary [B, R_cap, G, 64].

    Returns fp32 scores [rows, G, R_cap] (NaN where j >= floor(p/8))."""
    q8 = _c(q8, np.uint8)
    rows, H, _ = q8.shape
    summary = _c(summary, np.uint8)
    B, R_cap, G, _ = summary.shape
    w = _c(w_head, np.float32)
    w_stride = 0 if w.ndim == 1 else w.shape[1]
    out = np.full((rows, G, R_cap), np.nan, np.float32)
    rc = lib().o_score(_p(q8), H, G, _p(w), w_stride, _p(_c(row_seq, np.int32)),
                       _p(_c(row_pos, np.int64)), rows, _p(summary), B, R_cap, R_cap * G * IDX_DIM,
                       _p(out), nthreads or default_threads())
    if rc:
        raise ValueError("oracle score rejected its arguments")
    return out


def select(scores, row_pos, topk=512, nthreads=None):
    """scores [rows, G, R_cap] -> (ids int32 [rows, G, topk], scores fp32 [rows, G, topk])."""
    scores = _c(scores, np.float32)
    rows, G, R_cap = scores.shape
    ids = np.empty((rows, G, topk), np.int32)
    ss = np.empty((rows, G, topk), np.float32)
    rc = lib().o_select(_p(scores), _p(_c(row_pos, np.int64)), rows, G, R_cap, topk, _p(ids),
                        _p(ss), nthreads or default_threads())
    if rc:
        raise ValueError("oracle select rejected its arguments")
    return ids, ss


def attend(q16, k16, v16, sel, row_seq, row_pos, scale, nthreads=None):
    """q16 [rows, Hq, D]; k16, v16 [B, T_cap, Hkv, D]; sel int32 [rows, Hkv, topk].

    Returns (o fp64 [rows, Hq, D], lse fp64 [rows, Hq])."""
    q16 = _c(q16, np.uint16)
    rows, Hq, D = q16.shape
    k16 = _c(k16, np.uint16)
    v16 = _c(v16, np.uint16)
    B, T_cap, Hkv, D2 = k16.shape
    assert D2 == D and v16.shape == k16.shape
    sel = _c(sel, np.int32)
    topk = sel.shape[2]
    out = np.empty((rows, Hq, D), np.float64)
    lse = np.empty((rows, Hq), np.float64)
    rc = lib().o_attend(_p(q16), Hq * D, Hq, Hkv, D, _p(k16), _p(v16), T_cap * Hkv * D, Hkv * D,
                        T_cap, _p(sel), topk, _p(_c(row_seq, np.int32)), _p(_c(row_pos, np.int64)),
                        rows, float(scale), _p(out), _p(lse), nthreads or default_threads())
    if rc:
        raise ValueError("oracle attend rejected its arguments")
    return out, lse


# ---- fused projection [VLLM-proj] ---------------------------------------------

# Column blocks of the fused weight, in the order of its rows: the main
# attention's q, k, v, then the indexer's q, k, z, then the gate.
PROJ_PARTS = ("q", "k", "v", "index_q", "index_k", "index_z", "gate")


def proj_sizes(q_heads=16, kv_heads=4, head_dim=128, idx_heads=16, groups=4, idx_dim=64,
               gate=16):
    """Columns of each part (PROJ_PARTS order). The gate is per query head:
    one column per head by default."""
    return (q_heads * head_dim, kv_heads * head_dim, kv_heads * head_dim, idx_heads * idx_dim,
            groups * idx_dim, groups * idx_dim, gate)


def project(hidden16, w16, sizes, nthreads=None):
    """hidden16 bf16 [rows, H]; w16 bf16 [N, H] with N = sum(sizes).

    Returns (out fp64 [rows, N], {part: fp64 [rows, size]}) where the parts
    are consecutive column ranges of out in PROJ_PARTS order."""
    hidden16 = _c(hidden16, np.uint16)
    w16 = _c(w16, np.uint16)
    rows, H = hidden16.shape
    N, H2 = w16.shape
    assert H2 == H and N == sum(sizes) and len(sizes) == len(PROJ_PARTS)
    out = np.empty((rows, N), np.float64)
    rc = lib().o_project(_p(hidden16), rows, H, _p(w16), N, _p(out),
                         nthreads or default_threads())
    if rc:
        raise ValueError("oracle project rejected its arguments")
    parts, c0 = {}, 0
    for name, n in zip(PROJ_PARTS, sizes):
        parts[name] = out[:, c0:c0 + n]
        c0 += n
    return out, parts
