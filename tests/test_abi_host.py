"""The C ABI on the host (no GPU needed): the library loads, exports every
entry point include/step5.h declares, and rejects bad arguments with the
documented status before anything reaches the HIP runtime (a call that got as
far as a launch would return STEP5_E_HIP here, where there is no GPU).
Rejection rules follow the geometry checks of vLLM's Step-5 model page
(_validate_step5_dsa_parallel_geometry) and the header's argument contract.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "step5.h")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, 1, 2, 3, 4
A = 0x10000  # an aligned fake device address; never dereferenced by a rejected call


@pytest.fixture(scope="module")
def s5():
    import long_context_sparse_indexer_amd as m
    if not os.path.exists(m.LIB_PATH):
        from long_context_sparse_indexer_amd import _build
        _build.build()
    m.lib()
    return m


def geom(s5, **kw):
    g = s5.Step5Geom(16, 4, 64, 32, 8, 512, 16, 4, 128)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def test_exports_every_declared_symbol(s5):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(step5_\w+)\s*\(", text, re.M))
    assert {"step5_index_summarize", "step5_index_append", "step5_index_score_topk", "step5_sparse_attn",
            "step5_index_score_topk_workspace", "step5_sparse_attn_workspace",
            "step5_qkv_index_project", "step5_status_str", "step5_index_append_score_topk"} <= declared
    nm = subprocess.run(["nm", "-D", "--defined-only", s5.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (step5_\w+)$", nm, re.M))
    assert declared == exported
    for name in declared:
        assert hasattr(s5.lib(), name)


def test_status_strings(s5):
    assert s5.step5_status_str(0) == "ok"
    for c in (1, 2, 3, 4):
        assert s5.step5_status_str(c) != "unknown status"
    assert s5.step5_status_str(99) == "unknown status"


@pytest.mark.parametrize("kw,code", [
    ({}, OK),
    ({"groups": 2}, E_INVALID),                 # groups != kv_heads
    ({"idx_heads": 18}, E_INVALID),             # indexer heads do not divide into groups
    ({"q_heads": 8}, E_INVALID),                # 2 query heads per KV head
    ({"q_heads": 12}, E_INVALID),               # 3 per KV head
    ({"rope_dim": 33}, E_INVALID),
    ({"topk": 0}, E_INVALID),
    ({"q_heads": 32}, OK),                      # 8 per KV head
    ({"q_heads": 64}, OK),                      # 16 per KV head
    ({"head_dim": 192}, OK),
    ({"q_heads": 64, "head_dim": 192}, OK),     # Step-5's own layer shape
    ({"head_dim": 256}, E_UNSUPPORTED),
    ({"head_dim": 64}, E_UNSUPPORTED),
    ({"groups": 8, "kv_heads": 8, "q_heads": 32}, E_UNSUPPORTED),  # valid rules, 8 groups not built
    ({"topk": 256}, E_UNSUPPORTED),
])
def test_geometry_rules(s5, kw, code):
    g = geom(s5, **kw)
    L = s5.lib()
    # B = 0 is an empty call: with good geometry it succeeds without touching the GPU
    st = L.step5_index_summarize(C.byref(g), None, None, 0, 0, 0, 0, 0, None, None, 1e-6,
                                 None, 0, None, 0, 0, None)
    assert st == code
    assert L.step5_index_summarize(None, None, None, 0, 0, 0, 0, 0, None, None, 1e-6, None, 0,
                                   None, 0, 0, None) == E_INVALID


def _summ(s5, **over):
    g = geom(s5)
    a = dict(k=A, z=A, B=2, T=64, t0=0, sb=64 * 256, st=256, lnw=A, lnb=A, eps=1e-6, rope=A,
             rope_rows=64, summary=A, ssb=8 * 256, R_cap=8)
    a.update(over)
    return s5.lib().step5_index_summarize(
        C.byref(g), a["k"], a["z"], a["B"], a["T"], a["t0"], a["sb"], a["st"], a["lnw"],
        a["lnb"], a["eps"], a["rope"], a["rope_rows"], a["summary"], a["ssb"], a["R_cap"], None)


@pytest.mark.parametrize("over,code", [
    ({"t0": 4}, E_INVALID),
    ({"t0": -8}, E_INVALID),
    ({"B": -1}, E_INVALID),
    ({"T": -8}, E_INVALID),
    ({"T": 7}, OK),                 # no completed region: nothing to do
    ({"B": 0}, OK),
    ({"k": None}, E_INVALID),
    ({"z": A + 8}, E_INVALID),      # misaligned
    ({"lnw": None}, E_INVALID),
    ({"rope": None}, E_INVALID),
    ({"summary": A + 4}, E_INVALID),
    ({"st": 255}, E_INVALID),
    ({"st": 260}, E_INVALID),       # not a multiple of 8
    ({"sb": 64 * 256 - 8}, E_INVALID),
    ({"eps": 0.0}, E_INVALID),
    ({"eps": float("nan")}, E_INVALID),
    ({"rope_rows": 63}, E_INVALID),
    ({"R_cap": 7}, E_INVALID),
    ({"t0": 8, "rope_rows": 72}, E_INVALID),   # regions 1..8 need R_cap >= 9
    ({"ssb": 8 * 256 - 16}, E_INVALID),
    ({"ssb": 8 * 256 + 8}, E_INVALID),
])
def test_summarize_rejections(s5, over, code):
    assert _summ(s5, **over) == code


def _append(s5, **over):
    g = geom(s5)
    a = dict(k=A, z=A, ns=256, seq=A, pos=A, rows=16, kr=A, zr=A, B=16, slots=520,
             rsb=520 * 256, lnw=A, lnb=A, eps=1e-6, rope=A, rope_rows=131072, summary=A,
             ssb=16384 * 256, R_cap=16384)
    a.update(over)
    return s5.lib().step5_index_append(
        C.byref(g), a.get("flags", 0), a["k"], a["z"], a["ns"], a["seq"], a["pos"], a["rows"], a["kr"], a["zr"],
        a["B"], a["slots"], a["rsb"], a["lnw"], a["lnb"], a["eps"], a["rope"], a["rope_rows"],
        a["summary"], a["ssb"], a["R_cap"], None)


@pytest.mark.parametrize("over,code", [
    ({"rows": 0}, OK),
    ({"rows": 0, "k": None}, OK),    # an empty call touches nothing
    ({"rows": -1}, E_INVALID),
    ({"k": None}, E_INVALID),
    ({"seq": None}, E_INVALID),
    ({"zr": None}, E_INVALID),
    ({"summary": None}, E_INVALID),
    ({"z": A + 8}, E_INVALID),       # misaligned
    ({"kr": A + 2}, E_INVALID),
    ({"pos": A + 4}, E_INVALID),     # int64 array not 8-byte aligned
    ({"ns": 255}, E_INVALID),
    ({"ns": 260}, E_INVALID),        # not a multiple of 8
    ({"B": 0}, E_INVALID),
    ({"slots": 4}, E_INVALID),       # shorter than a region
    ({"slots": 524}, E_INVALID),     # not a multiple of the region
    ({"rsb": 520 * 256 - 8}, E_INVALID),
    ({"eps": -1.0}, E_INVALID),
    ({"rope_rows": 7}, E_INVALID),
    ({"R_cap": 0}, E_INVALID),
    ({"ssb": 16384 * 256 - 16}, E_INVALID),
    ({"ssb": 16384 * 256 + 8}, E_INVALID),
    ({"flags": 2}, E_INVALID),       # unknown flag bit
    ({"flags": 1, "k": None}, E_INVALID),
    ({"head_dim": 256}, E_UNSUPPORTED),
])
def test_append_rejections(s5, over, code):
    if "head_dim" in over:
        g = geom(s5, head_dim=over.pop("head_dim"))
        assert s5.lib().step5_index_append(C.byref(g), 0, A, A, 256, A, A, 16, A, A, 16, 520,
                                           520 * 256, A, A, 1e-6, A, 131072, A, 16384 * 256,
                                           16384, None) == code
        return
    assert _append(s5, **over) == code


def _score(s5, **over):
    g = geom(s5)
    rows = over.pop("rows", 4)
    R_cap = over.pop("R_cap", 64)
    need = s5.lib().step5_index_score_topk_workspace(C.byref(g), rows, R_cap)
    a = dict(flags=0, q=A, qs=1024, qw=A, eps=1e-6, rope=A, rope_rows=1024, w=A, ws_row=0,
             seq=A, pos=A, summary=A, B=1, ssb=R_cap * 256, ids=A, scores=None, ws=A, wsb=need)
    a.update(over)
    return s5.lib().step5_index_score_topk(
        C.byref(g), a["flags"], a["q"], a["qs"], a["qw"], a["eps"], a["rope"], a["rope_rows"],
        a["w"], a["ws_row"], a["seq"], a["pos"], rows, a["summary"], a["B"], R_cap, a["ssb"],
        a["ids"], a["scores"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    ({"rows": 0}, OK),
    ({"rows": -1}, E_INVALID),
    ({"flags": 2}, E_INVALID),
    ({"q": None}, E_INVALID),
    ({"qs": 1000}, E_INVALID),
    ({"qw": None}, E_INVALID),
    ({"flags": 1, "qw": None, "rope": None, "qs": 1024}, E_WORKSPACE),   # prepared q needs no prep args
    ({"flags": 1, "qs": 1032}, E_INVALID),                                # e4m3 rows 16-byte aligned
    ({"eps": -1.0}, E_INVALID),
    ({"rope_rows": 0}, E_INVALID),
    ({"w": None}, E_INVALID),
    ({"ws_row": 8}, E_INVALID),
    ({"seq": None}, E_INVALID),
    ({"pos": A + 4}, E_INVALID),
    ({"summary": None}, E_INVALID),
    ({"B": 0}, E_INVALID),
    ({"B": 2, "ssb": 63 * 256}, E_INVALID),
    ({"R_cap": 524289}, E_UNSUPPORTED),
    ({"R_cap": 0}, E_INVALID),
    ({"ids": None}, E_INVALID),
    ({"ws": None}, E_WORKSPACE),
    ({"ws": A + 128}, E_WORKSPACE),
    ({"rows": 300000}, E_UNSUPPORTED),
])
def test_score_topk_rejections(s5, over, code):
    if over.get("flags") == 1 and "wsb" not in over:
        over["wsb"] = 0          # then the call stops at the workspace check
    assert _score(s5, **over) == code


def _fused(s5, ap_over=None, **over):
    """step5_index_append_score_topk with valid arguments but those in
    `over` (score part) and `ap_over` (append part); ap_over=False passes no
    append struct."""
    g = geom(s5)
    rows = over.pop("rows", 4)
    R_cap = over.pop("R_cap", 64)
    need = s5.lib().step5_index_score_topk_workspace(C.byref(g), rows, R_cap)
    a = dict(flags=0, q=A, qs=1024, qw=A, eps=1e-6, rope=A, rope_rows=1024, w=A, ws_row=0,
             seq=A, pos=A, summary=A, B=1, ssb=R_cap * 256, ids=A, scores=None, ws=A, wsb=need)
    a.update(over)
    ap = None
    if ap_over is not False:
        f = dict(k_new=A, z_new=A, new_stride_row=256, k_ring=A, z_ring=A, ring_slots=520,
                 ring_stride_b=520 * 256, ln_w=A, ln_b=A, ln_eps=1e-6)
        f.update(ap_over or {})
        ap = C.byref(s5.Step5AppendIn(**f))
    return s5.lib().step5_index_append_score_topk(
        C.byref(g), a["flags"], ap, a["q"], a["qs"], a["qw"], a["eps"], a["rope"],
        a["rope_rows"], a["w"], a["ws_row"], a["seq"], a["pos"], rows, a["summary"], a["B"],
        R_cap, a["ssb"], a["ids"], a["scores"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("ap_over,over,code", [
    (None, {"rows": 0}, OK),
    (False, {}, E_INVALID),                                  # no append struct
    ({"k_new": None}, {}, E_INVALID),
    ({"ring_slots": 4}, {}, E_INVALID),
    ({"new_stride_row": 200}, {}, E_INVALID),
    ({"ln_eps": 0.0}, {}, E_INVALID),
    (None, {"flags": 1, "rope": None, "qw": None}, E_INVALID),  # the append needs rope
    (None, {"ids": None}, E_INVALID),
    (None, {"rows": -1}, E_INVALID),
    (None, {"R_cap": 524289}, E_UNSUPPORTED),
    (None, {"ws": None}, E_WORKSPACE),
    (None, {"wsb": 0}, E_WORKSPACE),
])
def test_append_score_topk_rejections(s5, ap_over, over, code):
    assert _fused(s5, ap_over, **over) == code


def test_append_score_topk_unsupported_geometry(s5):
    g = geom(s5, head_dim=256)
    f = s5.Step5AppendIn(A, A, 256, A, A, 520, 520 * 256, A, A, 1e-6)
    assert s5.lib().step5_index_append_score_topk(
        C.byref(g), 0, C.byref(f), A, 1024, A, 1e-6, A, 1024, A, 0, A, A, 4, A, 1, 64, 64 * 256,
        A, None, A, 1 << 20, None) == E_UNSUPPORTED


def test_score_topk_workspace_too_small(s5):
    g = geom(s5)
    need = s5.lib().step5_index_score_topk_workspace(C.byref(g), 4, 64)
    assert need > 0 and need % 256 == 0
    assert _score(s5, wsb=need - 1) == E_WORKSPACE


def test_workspace_sizes(s5):
    L = s5.lib()
    g = geom(s5)
    assert L.step5_index_score_topk_workspace(C.byref(g), 0, 100) == 0
    assert L.step5_index_score_topk_workspace(C.byref(g), 4, 0) == 0
    assert L.step5_index_score_topk_workspace(C.byref(geom(s5, groups=2)), 4, 64) == 0
    # q8 (rows*1024) + bounds (rows*4*R_cap*8), 256-aligned, plus chunk lists and
    # counters; more than 64 rows over at most 4,096 regions select with fused
    # intervals: no bounds
    w1 = L.step5_index_score_topk_workspace(C.byref(g), 2048, 4096)
    assert 2048 * 1024 <= w1 < 2048 * 1024 + 2048 * 4 * 8 + 4096
    w2 = L.step5_index_score_topk_workspace(C.byref(g), 2048, 4097)
    assert w2 >= 2048 * 1024 + 2048 * 4 * 4097 * 8
    w4 = L.step5_index_score_topk_workspace(C.byref(g), 16, 16384)
    assert w4 >= 16 * 1024 + 16 * 4 * 16384 * 8                       # one pass: no chunk lists
    w5 = L.step5_index_score_topk_workspace(C.byref(g), 1, 131072)
    assert w5 >= 1024 + 4 * 131072 * 8 + 4 * 8 * 512 * 8               # 8 chunk lists of 512
    assert L.step5_sparse_attn_workspace(C.byref(g), 2048) == 0          # prefill: unsplit
    assert L.step5_sparse_attn_workspace(C.byref(g), 16) > 0             # decode: split states
    assert L.step5_sparse_attn_workspace(C.byref(g), 0) == 0


def _attn(s5, **over):
    g = geom(s5)
    rows = over.pop("rows", 16)
    need = s5.lib().step5_sparse_attn_workspace(C.byref(g), rows)
    a = dict(q=A, qs=2048, k=A, v=A, B=16, kvb=4096 * 512, kvt=512, T=4096, sel=A, seq=A, pos=A,
             scale=0.088, out=A, lse=None, ws=A, wsb=need)
    a.update(over)
    return s5.lib().step5_sparse_attn(
        C.byref(g), a["q"], a["qs"], a["k"], a["v"], a["B"], a["kvb"], a["kvt"], a["T"], a["sel"],
        a["seq"], a["pos"], rows, a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    ({"rows": 0}, OK),
    ({"rows": -3}, E_INVALID),
    ({"q": None}, E_INVALID),
    ({"qs": 2040}, E_INVALID),
    ({"k": A + 2}, E_INVALID),
    ({"v": None}, E_INVALID),
    ({"B": 0}, E_INVALID),
    ({"T": 0}, E_INVALID),
    ({"kvt": 500}, E_INVALID),
    ({"kvb": 4095 * 512}, E_INVALID),
    ({"sel": None}, E_INVALID),
    ({"pos": None}, E_INVALID),
    ({"scale": 0.0}, E_INVALID),
    ({"scale": float("inf")}, E_INVALID),
    ({"scale": float("nan")}, E_INVALID),
    ({"out": None}, E_INVALID),
    ({"lse": A + 2}, E_INVALID),
    ({"ws": None}, E_WORKSPACE),
    ({"wsb": 16}, E_WORKSPACE),
])
def test_sparse_attn_rejections(s5, over, code):
    assert _attn(s5, **over) == code


@pytest.mark.parametrize("over,code", [
    ({"rows": 0}, OK),
    ({"rows": -3}, E_INVALID),
    ({"q": None}, E_INVALID),
    ({"qs": 2040}, E_INVALID),
    ({"k": A + 2}, E_INVALID),
    ({"T": 0}, E_INVALID),
    ({"sel": None}, E_INVALID),
    ({"scale": float("nan")}, E_INVALID),
    ({"out": None}, E_INVALID),
])
def test_sparse_attn_noalloc_rejections(s5, over, code):
    """The allocation-free attention call checks the same arguments before any
    HIP call (here, with no GPU, a call that passed them would fail later)."""
    g = over.pop("g", geom(s5))
    rows = over.pop("rows", 16)
    a = dict(q=A, qs=2048, k=A, v=A, B=16, kvb=4096 * 512, kvt=512, T=4096, sel=A, seq=A, pos=A,
             scale=0.088, out=A, lse=None)
    a.update(over)
    assert s5.lib().step5_sparse_attn_noalloc(
        C.byref(g), a["q"], a["qs"], a["k"], a["v"], a["B"], a["kvb"], a["kvt"], a["T"], a["sel"],
        a["seq"], a["pos"], rows, a["scale"], a["out"], a["lse"], None) == code


def test_sparse_attn_static_scratch_covers_every_geometry(s5):
    """The static scratch (16 MiB) holds the split states of every accepted
    geometry at every row count."""
    L = s5.lib()
    worst = 0
    for hq, hd in ((16, 128), (32, 128), (64, 128), (16, 192), (32, 192), (64, 192)):
        g = geom(s5, q_heads=hq, head_dim=hd)
        for rows in list(range(1, 300)) + [1000, 4096, 65536]:
            worst = max(worst, L.step5_sparse_attn_workspace(C.byref(g), rows))
    assert 0 < worst <= 16 << 20


def test_sparse_attn_geometry_strides_and_workspace(s5):
    """16 query heads per KV head of 192 dims: q rows need 64 x 192 elements,
    K/V token rows 4 x 192, and the split states grow with the heads and dims."""
    L = s5.lib()
    g = geom(s5, q_heads=64, head_dim=192)
    need = L.step5_sparse_attn_workspace(C.byref(g), 16)
    assert need >= 16 * 4 * 2 * 16 * 194 * 4        # at least 2 splits of 16 heads x (m, l, o)
    assert need > L.step5_sparse_attn_workspace(C.byref(geom(s5)), 16)

    def call(qs, kvt):
        return L.step5_sparse_attn(C.byref(g), A, qs, A, A, 16, 4096 * kvt, kvt, 4096, A, A, A, 16,
                                   0.072, A, None, None if need == 0 else A, need, None)
    assert call(64 * 192 - 8, 4 * 192) == E_INVALID
    assert call(64 * 192, 4 * 192 - 8) == E_INVALID
    assert L.step5_sparse_attn(C.byref(g), A, 64 * 192, A, A, 16, 4096 * 768, 768, 4096, A, A, A,
                               16, 0.072, A, None, A, need - 1, None) == E_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import long_context_sparse_indexer_amd as m
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(ImportError):
        m.lib()


def test_fused_call_rejects_rows_sharing_a_sequence(s5):
    """check_distinct: two rows naming one sequence are rejected by the binding
    before anything reaches the library (the library cannot see device
    values); distinct rows pass the check and go on to the argument checks."""
    import torch
    rows = 3
    bf = dict(dtype=torch.bfloat16)
    k_new, z_new = torch.zeros(rows, 4, 64, **bf), torch.zeros(rows, 4, 64, **bf)
    ring = torch.zeros(4, 16, 4, 64, **bf)
    S = torch.zeros(4, 100, 4, 64, dtype=torch.uint8)
    args = (k_new, z_new, ring, ring.clone(), torch.ones(64), torch.zeros(64), 1e-6,
            torch.zeros(rows, 16, 64, **bf), torch.ones(16))
    pos = torch.full((rows,), 40, dtype=torch.int64)
    ids = torch.zeros(rows, 4, 512, dtype=torch.int32)
    with pytest.raises(ValueError, match="share a sequence"):
        s5.step5_index_append_score_topk(*args, torch.tensor([0, 2, 0], dtype=torch.int32), pos, S,
                                         ids, rope=torch.zeros(800, 32, **bf),
                                         q_norm_w=torch.zeros(64), check_distinct=True)


# ---- fused projection --------------------------------------------------------

def _proj(s5, widths=(2048, 512, 512, 1024, 256, 256, 16), **over):
    g = over.pop("g", geom(s5))
    a = dict(h=A, hs=4096, rows=16, H=4096, w=A, gate=widths[6])
    a.update(over)
    outs = (s5.Step5ProjOut * 7)()
    for i, wdt in enumerate(widths):
        outs[i].ptr = over.get(f"out{i}", A)
        outs[i].stride_row = over.get(f"stride{i}", wdt)
    return s5.lib().step5_qkv_index_project(C.byref(g), a["h"], a["hs"], a["rows"], a["H"], a["w"],
                                            a["gate"], outs, None)


@pytest.mark.parametrize("over,code", [
    ({"rows": 0}, OK),
    ({"rows": -1}, E_INVALID),
    ({"h": None}, E_INVALID),
    ({"h": A + 8}, E_INVALID),
    ({"hs": 4088}, E_INVALID),
    ({"hs": 4100}, E_INVALID),
    ({"w": None}, E_INVALID),
    ({"w": A + 2}, E_INVALID),
    ({"H": 0}, E_INVALID),
    ({"H": 4032, "hs": 4096}, E_UNSUPPORTED),   # not a multiple of 128
    ({"gate": -16}, E_INVALID),
    ({"out0": None}, E_INVALID),
    ({"out3": A + 4}, E_INVALID),
    ({"stride1": 504}, E_INVALID),
    ({"stride5": 260}, E_INVALID),
    ({"g": None}, E_INVALID),
])
def test_project_rejections(s5, over, code):
    if "g" in over and over["g"] is None:
        outs = (s5.Step5ProjOut * 7)()
        assert s5.lib().step5_qkv_index_project(None, A, 4096, 16, 4096, A, 16, outs, None) == code
        return
    assert _proj(s5, **over) == code


def test_project_gate_and_geometry(s5):
    """A gate of 24 columns is not a multiple of 16 (unsupported); a gate of
    0 leaves the seventh output untouched (its pointer may be null); the
    16-heads-per-KV-head x 192 geometry widens q, k and v."""
    assert _proj(s5, widths=(2048, 512, 512, 1024, 256, 256, 24), rows=0) == E_UNSUPPORTED
    assert _proj(s5, widths=(2048, 512, 512, 1024, 256, 256, 0), out6=None, rows=0) == OK
    g = geom(s5, q_heads=64, head_dim=192)
    assert _proj(s5, widths=(64 * 192, 768, 768, 1024, 256, 256, 64), g=g, rows=0) == OK
    assert _proj(s5, widths=(64 * 192, 768, 768, 1024, 256, 256, 64), g=g, stride0=64 * 192 - 8,
                 rows=0) == E_INVALID
    assert _proj(s5, g=geom(s5, topk=256), rows=0) == E_UNSUPPORTED
