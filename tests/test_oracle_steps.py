"""Pins of the oracle's steps against facts that do not run through it:
special cases with closed forms, the fp64 textbook definitions within their
rounding bounds, brute force on tiny inputs, hand-worked fixtures, and the
dense attention that the sparse path must equal while every region is
selected.

Sources: TensorFold pull request #903 "Step-5-Preview on one 256 GB Mac"
(indexer commit note: the arithmetic of every step; first commit note: dense
attention is exact while the indexer selects every region).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rope_f64(y, cs_row16):
    """fp64 NEOX rotation with the table's (bf16) cos/sin values."""
    cs = _f(cs_row16).astype(np.float64)
    c, s = cs[..., :16], cs[..., 16:]
    a, b = y[..., :16].copy(), y[..., 16:32].copy()
    out = y.copy()
    out[..., :16] = a * c - b * s
    out[..., 16:32] = b * c + a * s
    return out


# ---- rope table (input) ----------------------------------------------------

def test_rope_table_is_bf16_of_cos_sin():
    tab = W.rope_table(4096)
    assert tab.shape == (4096, 32) and tab.dtype == torch.bfloat16
    t = tab.float().numpy().astype(np.float64)
    p = np.arange(4096, dtype=np.float64)[:, None]
    inv = 10000.0 ** (-np.arange(0, 32, 2) / 32.0)
    ang = p * inv[None, :]
    # bf16 rounding (2^-9 relative) plus the fp32 angle's rounding (p * 2^-24)
    tol = 2.0 ** -8 + 4096 * 2.0 ** -23
    assert np.abs(t[:, :16] - np.cos(ang)).max() <= tol
    assert np.abs(t[:, 16:] - np.sin(ang)).max() <= tol
    assert np.all(t[0, :16] == 1.0) and np.all(t[0, 16:] == 0.0)


# ---- sum64 ---------------------------------------------------------------

def test_sum64_exact_on_integers_and_within_pairwise_bound(orc):
    rng = np.random.default_rng(17)
    for _ in range(200):
        x = rng.integers(-1000, 1000, 64).astype(np.float32)
        assert orc.sum64(x) == float(x.astype(np.int64).sum())
    for _ in range(2000):
        x = (rng.standard_normal(64) * np.exp(rng.uniform(-8, 8, 64))).astype(np.float32)
        exact = math.fsum(x.astype(np.float64))
        bound = 6 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum() * (1 + 1e-6)
        assert abs(orc.sum64(x) - exact) <= bound
    # one dropped term anywhere would show here
    for i in range(64):
        x = np.zeros(64, np.float32)
        x[i] = 1.0
        assert orc.sum64(x) == 1.0


# ---- k prep: LayerNorm with bias, NEOX rotation, bf16 --------------------

def _params(seed):
    g = torch.Generator().manual_seed(seed)
    ln_w = (torch.rand(64, generator=g) + 0.5).numpy()
    ln_b = (torch.rand(64, generator=g) - 0.5).numpy()
    qw = (torch.rand(64, generator=g) - 0.5).numpy()
    return ln_w, ln_b, qw


def test_k_prep_constant_vector_gives_bias(orc):
    ln_w, ln_b, _ = _params(17)
    rope = _bf(np.tile(np.r_[np.ones(16), np.zeros(16)], (4, 1)))   # identity rotation
    for c in (0.0, 1.0, -3.5, 1000.0):
        x = _bf(np.full((1, 64), c))
        out = orc.k_prep(x, ln_w, ln_b, EPS, rope, np.array([0]))
        assert np.array_equal(out[0], _f(_bf(ln_b)))


def test_k_prep_matches_fp64_definition(orc):
    ln_w, ln_b, _ = _params(41)
    rope = W.rope_table(6000).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(41)
    n = 4000
    x16 = _bf(rng.standard_normal((n, 64)) * rng.uniform(0.1, 10, (n, 1)))
    pos = rng.integers(0, 6000, n)
    got = orc.k_prep(x16, ln_w, ln_b, EPS, rope, pos).astype(np.float64)
    x = _f(x16).astype(np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = (x - mu) / np.sqrt(var + EPS) * ln_w.astype(np.float64) + ln_b.astype(np.float64)
    y = _rope_f64(y, rope[pos])
    # one bf16 rounding (2^-9 relative) plus a few fp32 roundings
    assert np.all(np.abs(got - y) <= 2.0 ** -8 * np.abs(y) + 1e-5)


def test_k_prep_position_zero_is_unrotated(orc):
    ln_w, ln_b, _ = _params(17)
    rope = W.rope_table(8).view(torch.int16).numpy().view(np.uint16)
    ident = _bf(np.tile(np.r_[np.ones(16), np.zeros(16)], (8, 1)))
    x16 = _bf(np.random.default_rng(1).standard_normal((50, 64)))
    a = orc.k_prep(x16, ln_w, ln_b, EPS, rope, np.zeros(50, np.int64))
    b = orc.k_prep(x16, ln_w, ln_b, EPS, ident, np.zeros(50, np.int64))
    assert np.array_equal(a, b)


def test_rotation_preserves_pair_norms_and_relative_position(orc):
    """q(p).k(p') after rotation depends on p - p' only (fp64, bf16 table)."""
    rope = W.rope_table(2048).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(3)
    a = rng.standard_normal(64)
    b = rng.standard_normal(64)
    dots = [(_rope_f64(a, rope[p]) @ _rope_f64(b, rope[p - 5])) for p in (5, 100, 1000, 2000)]
    assert max(dots) - min(dots) < 0.05 * np.abs(a).sum() * np.abs(b).sum() / 64
    r = _rope_f64(a, rope[777])
    n0 = a[:16] ** 2 + a[16:32] ** 2
    n1 = r[:16] ** 2 + r[16:32] ** 2
    assert np.allclose(n0, n1, rtol=2e-2)


# ---- q prep: RMSNorm (1 + w), rotation, bf16, e4m3 -----------------------

def test_q_prep_zero_and_constant(orc):
    _, _, qw = _params(17)
    rope = W.rope_table(16).view(torch.int16).numpy().view(np.uint16)
    q = np.zeros((1, 16, 64), np.uint16)
    assert np.all(orc.e4m3_to_f64(orc.q_prep(q, qw, EPS, rope, np.array([3]))) == 0.0)
    # constant vector, w = 0, position 0: every entry is 1/sqrt(1 + eps/c^2) -> e4m3 1.0
    q = _bf(np.full((1, 16, 64), 2.5))
    assert np.all(orc.q_prep(q, np.zeros(64, np.float32), EPS, rope, np.array([0])) == 0x38)
    q = _bf(np.full((1, 16, 64), -2.5))
    assert np.all(orc.q_prep(q, np.zeros(64, np.float32), EPS, rope, np.array([0])) == 0xB8)


def test_q_prep_matches_fp64_definition(orc):
    _, _, qw = _params(41)
    rope = W.rope_table(6000).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(5)
    rows = 64
    q16 = _bf(rng.standard_normal((rows, 16, 64)))
    pos = rng.integers(0, 6000, rows)
    got = orc.e4m3_to_f64(orc.q_prep(q16, qw, EPS, rope, pos))
    x = _f(q16).astype(np.float64)
    y = x / np.sqrt((x ** 2).mean(axis=2, keepdims=True) + EPS) * (1.0 + qw.astype(np.float64))
    y = _rope_f64(y, rope[pos][:, None, :])
    # e4m3 keeps 3 mantissa bits: within half a step (2^-4 relative) plus bf16 double rounding
    tol = 2.0 ** -4 * np.abs(y) * (1 + 2.0 ** -7) + 2.0 ** -10
    assert np.all(np.abs(got - y) <= tol)


# ---- region summary --------------------------------------------------------

def _summary_inputs(seed, B=2, T=64, t0=0):
    ln_w, ln_b, _ = _params(seed)
    rng = np.random.default_rng(seed)
    k16 = _bf(rng.standard_normal((B, T, 4, 64)))
    z16 = _bf(rng.standard_normal((B, T, 4, 64)) * 2)
    rope = W.rope_table(t0 + T + 8).view(torch.int16).numpy().view(np.uint16)
    return k16, z16, ln_w, ln_b, rope


def _kp_of(orc, k16, ln_w, ln_b, rope, t0):
    B, T, G, _ = k16.shape
    pos = np.broadcast_to((t0 + np.arange(T))[None, :, None], (B, T, G)).reshape(-1)
    return orc.k_prep(k16.reshape(-1, 64), ln_w, ln_b, EPS, rope, pos).reshape(B, T, G, 64)


def test_summary_constant_z_is_mean_of_k(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(17)
    z16[:] = _bf(np.full(z16.shape, 0.75))
    S = orc.summarize(k16, z16, 0, ln_w, ln_b, EPS, rope)
    kp = _kp_of(orc, k16, ln_w, ln_b, rope, 0).astype(np.float64)
    mean = kp.reshape(2, 8, 8, 4, 64).mean(axis=2)
    got = orc.e4m3_to_f64(S)
    assert np.all(np.abs(got - mean) <= 2.0 ** -4 * np.abs(mean) * (1 + 2.0 ** -7) + 2.0 ** -10)


def test_summary_dominant_token_is_exactly_its_k(orc):
    """One token whose z beats the others by more than 88: its softmax
    weight is 1 and the rest vanish, so the summary is e4m3 of its k."""
    k16, z16, ln_w, ln_b, rope = _summary_inputs(41)
    rng = np.random.default_rng(9)
    zf = np.zeros(z16.shape, np.float32)
    win = rng.integers(0, 8, (2, 8, 4, 64))
    zr = zf.reshape(2, 8, 8, 4, 64)
    for t in range(8):
        zr[:, :, t][win == t] = 96.0
    z16[:] = _bf(zf)
    S = orc.summarize(k16, z16, 0, ln_w, ln_b, EPS, rope)
    kp = _kp_of(orc, k16, ln_w, ln_b, rope, 0).reshape(2, 8, 8, 4, 64)
    pick = np.take_along_axis(kp, win[:, :, None], axis=2)[:, :, 0]
    want = orc.bf16_to_e4m3(_bf(pick))
    assert np.array_equal(S, want)


def test_summary_weights_follow_z_not_minus_z(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(5, B=1, T=8)
    zf = np.zeros(z16.shape, np.float32)
    zf[0, 3] = 4.0                         # token 3 gets weight ~ e^4/(e^4 + 7)
    z16[:] = _bf(zf)
    S = orc.e4m3_to_f64(orc.summarize(k16, z16, 0, ln_w, ln_b, EPS, rope))[0, 0]
    kp = _kp_of(orc, k16, ln_w, ln_b, rope, 0)[0].astype(np.float64)
    w = np.ones(8)
    w[3] = math.exp(4.0)
    want = (w[:, None, None] * kp).sum(0) / w.sum()
    assert np.all(np.abs(S - want) <= 2.0 ** -4 * np.abs(want) * 1.01 + 2.0 ** -10)


def test_summary_convex_and_shadow_agreement(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(17, B=3, T=256, t0=64)
    S, sh = orc.summarize(k16, z16, 64, ln_w, ln_b, EPS, rope, shadow=True)
    S = S[:, 8:]
    sh = sh[:, 8:]
    kp = _kp_of(orc, k16, ln_w, ln_b, rope, 64).reshape(3, 32, 8, 4, 64)
    lo, hi = kp.min(axis=2), kp.max(axis=2)
    got = orc.e4m3_to_f64(S)
    assert np.all(got >= orc.e4m3_to_f64(orc.bf16_to_e4m3(_bf(lo))))
    assert np.all(got <= orc.e4m3_to_f64(orc.bf16_to_e4m3(_bf(hi))))
    assert np.all((sh >= lo - 1e-9) & (sh <= hi + 1e-9))
    # the fp32 pipeline rounds like exact arithmetic except at rare midpoints
    exact_route = orc.bf16_to_e4m3(_bf(sh))
    assert np.mean(exact_route != S) < 2e-3
    assert np.all(np.abs(got - sh) <= 2.0 ** -4 * np.abs(sh) * 1.01 + 2.0 ** -10)


def test_summary_only_writes_completed_regions(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(17, B=1, T=21, t0=16)
    base = np.full((1, 8, 4, 64), 0x55, np.uint8)
    S = orc.summarize(k16, z16, 16, ln_w, ln_b, EPS, rope, R_cap=8, summary=base.copy())
    # tokens 16..36: regions 2, 3 complete (16..31), region 4 open (32..36)
    assert np.all(S[:, :2] == 0x55) and np.all(S[:, 4:] == 0x55)
    assert not np.all(S[:, 2:4] == 0x55)
    with pytest.raises(ValueError):
        orc.summarize(k16, z16, 12, ln_w, ln_b, EPS, rope, R_cap=8)     # t0 not a region start


# ---- incremental cache update (k/z rings + summary on region completion) ----

def _stream(orc, k16, z16, ln_w, ln_b, rope, slots, chunks, R_cap):
    """Feed B sequences' tokens through orc.append in the given chunk sizes
    (every sequence the same chunk at once); returns rings and summary."""
    B, T = k16.shape[:2]
    k_ring = np.zeros((B, slots, 4, 64), np.uint16)
    z_ring = np.zeros((B, slots, 4, 64), np.uint16)
    S = np.full((B, R_cap, 4, 64), 0x55, np.uint8)
    t = 0
    for n in chunks:
        pos = np.repeat(np.arange(t, t + n)[None], B, 0).reshape(-1)
        seq = np.repeat(np.arange(B, dtype=np.int32)[:, None], n, 1).reshape(-1)
        orc.append(k16[:, t:t + n].reshape(-1, 4, 64), z16[:, t:t + n].reshape(-1, 4, 64), seq, pos,
                   k_ring, z_ring, ln_w, ln_b, EPS, rope, S)
        t += n
    assert t == T
    return k_ring, z_ring, S


@pytest.mark.parametrize("chunks", [[1] * 61, [5, 11, 16, 1, 7, 13, 8], [3, 17, 17, 17, 7]])
def test_append_equals_batch_summary(orc, chunks):
    """Tokens appended one at a time or in chunks (each within the ring's
    reach, slots - 7) leave exactly the summaries the batch summary writes
    from the contiguous k and z, and nothing for the open region."""
    k16, z16, ln_w, ln_b, rope = _summary_inputs(23, B=2, T=61)
    R_cap = 9
    _, _, S = _stream(orc, k16, z16, ln_w, ln_b, rope, slots=24, chunks=chunks, R_cap=R_cap)
    want = orc.summarize(k16, z16, 0, ln_w, ln_b, EPS, rope, R_cap=R_cap,
                         summary=np.full((2, R_cap, 4, 64), 0x55, np.uint8))
    assert np.array_equal(S, want)
    assert np.all(S[:, 7:] == 0x55)          # tokens 56..60 leave region 7 open


def test_append_ring_holds_latest_token_per_slot(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(5, B=1, T=40)
    k_ring, z_ring, _ = _stream(orc, k16, z16, ln_w, ln_b, rope, slots=16, chunks=[9, 9, 9, 9, 4],
                                R_cap=5)
    for i in range(16):
        last = max(p for p in range(40) if p % 16 == i)
        assert np.array_equal(k_ring[0, i], k16[0, last]) and np.array_equal(z_ring[0, i], z16[0, last])


def test_append_skips_invalid_rows(orc):
    k16, z16, ln_w, ln_b, rope = _summary_inputs(7, B=2, T=8)
    k_ring = np.zeros((2, 8, 4, 64), np.uint16)
    z_ring = np.zeros((2, 8, 4, 64), np.uint16)
    S = np.full((2, 1, 4, 64), 0x55, np.uint8)
    # sequence 2 does not exist, -1 is no sequence, position 8 is region 1 >= R_cap
    orc.append(k16[0, :3], z16[0, :3], np.array([2, -1, 0], np.int32), np.array([7, 7, 8]),
               k_ring, z_ring, ln_w, ln_b, EPS, rope, S)
    assert np.all(k_ring == 0) and np.all(z_ring == 0) and np.all(S == 0x55)


# ---- scores ----------------------------------------------------------------

def test_score_dyadic_closed_form(orc):
    """q8 and summaries from {+-1/4, +-1/2, +-1, +-2}, w_h = (h+1)/16: the
    score is a multiple of 1/256 computed here in Python integers."""
    rng = np.random.default_rng(17)
    codes = np.array(W.TIE_CODES, np.uint8)
    rows, R = 3, 40
    q8 = codes[rng.integers(0, 8, (rows, 16, 64))]
    S = codes[rng.integers(0, 8, (1, R, 4, 64))]
    w = np.arange(1, 17, dtype=np.float32) / 16
    pos = np.array([8 * R, 8 * R + 5, 8 * 17 + 3])
    got = orc.score(q8, w, np.zeros(rows, np.int32), pos, S)
    val4 = {0x28: 1, 0x30: 2, 0x38: 4, 0x40: 8}          # value * 4
    qi = np.vectorize(lambda c: (-1 if c & 0x80 else 1) * val4[c & 0x7F])(q8)
    si = np.vectorize(lambda c: (-1 if c & 0x80 else 1) * val4[c & 0x7F])(S[0])
    for r in range(rows):
        nc = pos[r] // 8
        assert np.all(np.isnan(got[r, :, nc:]))
        for g in range(4):
            for j in range(nc):
                tot = 0
                for hh in range(4):
                    h = 4 * g + hh
                    dot16 = int((qi[r, h].astype(np.int64) * si[j, g]).sum())   # dot * 16
                    tot += max(dot16, 0) * (h + 1)                           # * 256
                assert got[r, g, j] == tot / 256.0


def test_score_random_matches_fp64_and_negative_is_zero(orc):
    rng = np.random.default_rng(41)
    q8 = orc.bf16_to_e4m3(_bf(rng.standard_normal((2, 16, 64)) * 2))
    S = orc.bf16_to_e4m3(_bf(rng.standard_normal((2, 30, 4, 64))))
    w = rng.uniform(0, 1, 16).astype(np.float32)
    pos = np.array([239, 239])
    got = orc.score(q8, w, np.array([0, 1], np.int32), pos, S)
    qf, sf = orc.e4m3_to_f64(q8), orc.e4m3_to_f64(S)
    for r in range(2):
        d = np.einsum("hd,jgd->gjh", qf[r], sf[r])                  # [4, 30, 16]
        want = np.zeros((4, 29))
        for g in range(4):
            t = np.maximum(d[g, :29, 4 * g:4 * g + 4], 0)
            want[g] = t @ w[4 * g:4 * g + 4].astype(np.float64)
        assert np.allclose(got[r, :, :29], want, rtol=1e-6, atol=1e-7)
    # all dots negative -> exactly +0
    S2 = np.full((1, 4, 4, 64), 0x38, np.uint8)
    q2 = np.full((1, 16, 64), 0xB8, np.uint8)
    z = orc.score(q2, w, np.array([0], np.int32), np.array([31]), S2)
    assert np.all(z[0, :, :3] == 0) and not np.any(np.signbit(z[0, :, :3]))


def test_score_per_row_weights(orc):
    rng = np.random.default_rng(2)
    q8 = orc.bf16_to_e4m3(_bf(rng.standard_normal((2, 16, 64))))
    S = orc.bf16_to_e4m3(_bf(rng.standard_normal((1, 10, 4, 64))))
    w2 = rng.uniform(0, 1, (2, 16)).astype(np.float32)
    pos = np.array([80, 80])
    both = orc.score(q8, w2, np.zeros(2, np.int32), pos, S)
    for r in range(2):
        one = orc.score(q8[r:r + 1], w2[r], np.zeros(1, np.int32), pos[:1], S)
        assert np.array_equal(both[r], one[0], equal_nan=True)


# ---- selection -------------------------------------------------------------

def test_select_golden_ties(orc):
    with open(os.path.join(GOLDEN, "select_ties.json")) as fh:
        g = json.load(fh)
    s = np.array(g["scores"], np.float32)[None, None, :]
    for case in g["cases"]:
        ids, _ = orc.select(s, np.array([8 * s.shape[2]]), topk=case["topk"])
        assert ids[0, 0].tolist() == case["ids"]


def test_select_brute_force_tiny(orc):
    rng = np.random.default_rng(17)
    for trial in range(300):
        n = int(rng.integers(0, 40))
        k = int(rng.integers(1, 12))
        s = rng.choice(np.array([0.0, -0.0, 1.0, 1.5, 2.0, 3.25, 7.0], np.float32), n + 3)
        s = s if trial % 2 else rng.standard_normal(n + 3).astype(np.float32)
        ids, ss = orc.select(s[None, None, :], np.array([8 * n + int(rng.integers(0, 8))]), topk=k)
        want = sorted(range(n), key=lambda j: (-float(s[j]), j))[:k]
        want += [-1] * (k - len(want))
        assert ids[0, 0].tolist() == want
        for i, j in enumerate(want):
            if j >= 0:
                assert ss[0, 0, i] == s[j]


@pytest.mark.parametrize("ncand", [511, 512, 513])
def test_select_boundary(orc, ncand):
    rng = np.random.default_rng(ncand)
    s = rng.standard_normal((1, 4, 600)).astype(np.float32)
    ids, _ = orc.select(s, np.array([8 * ncand + 7]), topk=512)
    for g in range(4):
        want = sorted(range(ncand), key=lambda j: (-float(s[0, g, j]), j))[:512]
        got = ids[0, g].tolist()
        assert got[:len(want)] == want
        assert all(x == -1 for x in got[len(want):])
        if ncand <= 512:
            assert sorted(got[:ncand]) == list(range(ncand))


# ---- attention -------------------------------------------------------------

def _dense_causal(qf, kf, vf, p, scale):
    """Textbook attention of one row over tokens 0..p (fp64, numpy)."""
    lg = scale * (kf[: p + 1] @ qf)
    e = np.exp(lg - lg.max())
    return (e[:, None] * vf[: p + 1]).sum(0) / e.sum(), lg.max() + math.log(e.sum())


def _attn_inputs(seed, B, T, rows, D=128):
    rng = np.random.default_rng(seed)
    q = _bf(rng.standard_normal((rows, 16, D)))
    k = _bf(rng.standard_normal((B, T, 4, D)))
    v = _bf(rng.standard_normal((B, T, 4, D)))
    return q, k, v


def test_attend_all_selected_equals_dense_causal(orc):
    B, T = 3, 300
    q, k, v = _attn_inputs(17, B, T, 3)
    pos = np.array([299, 171, 9])
    seq = np.array([0, 1, 2], np.int32)
    sel = np.full((3, 4, 512), -1, np.int32)
    for r in range(3):
        nc = pos[r] // 8
        order = np.random.default_rng(r).permutation(nc)       # any order of the ids
        sel[r, :, :nc] = order[None, :]
    scale = 1 / math.sqrt(128)
    o, lse = orc.attend(q, k, v, sel, seq, pos, scale)
    qf, kf, vf = _f(q).astype(np.float64), _f(k).astype(np.float64), _f(v).astype(np.float64)
    for r in range(3):
        for h in range(16):
            want, wl = _dense_causal(qf[r, h], kf[seq[r], :, h // 4], vf[seq[r], :, h // 4], pos[r], scale)
            assert np.allclose(o[r, h], want, rtol=1e-12, atol=1e-12)
            assert abs(lse[r, h] - wl) < 1e-10


def test_attend_sparse_equals_masked_dense(orc):
    B, T = 1, 8 * 40 + 5
    q, k, v = _attn_inputs(41, B, T, 2)
    pos = np.array([T - 1, T - 3])
    rng = np.random.default_rng(0)
    sel = np.full((2, 4, 6), -1, np.int32)
    for r in range(2):
        for g in range(4):
            sel[r, g, :5] = rng.choice(40, 5, replace=False)
    scale = 0.1
    o, _ = orc.attend(q, k, v, sel, np.zeros(2, np.int32), pos, scale)
    qf, kf, vf = _f(q).astype(np.float64), _f(k).astype(np.float64), _f(v).astype(np.float64)
    for r in range(2):
        p = pos[r]
        for h in range(16):
            g = h // 4
            mask = np.zeros(T, bool)
            for j in sel[r, g]:
                if j >= 0:
                    mask[8 * j:8 * j + 8] = True
            mask[8 * (p // 8): p + 1] = True
            lg = scale * (kf[0, :, g] @ qf[r, h])
            lg[~mask] = -np.inf
            e = np.exp(lg - lg.max())
            want = (e[:, None] * vf[0, :, g]).sum(0) / e.sum()
            assert np.allclose(o[r, h], want, rtol=1e-12, atol=1e-12)


def test_attend_first_token_and_identical_keys(orc):
    q, k, v = _attn_inputs(5, 1, 64, 1)
    sel = np.full((1, 4, 512), -1, np.int32)
    o, lse = orc.attend(q, k, v, sel, np.zeros(1, np.int32), np.array([0]), 0.088)
    vf = _f(v).astype(np.float64)
    for h in range(16):
        assert np.array_equal(o[0, h], vf[0, 0, h // 4])
    # every key identical: the weights are uniform and o is the mean of V over the set
    k2 = k.copy()
    k2[:] = k[0, 0][None, None]
    sel[0, :, :3] = np.array([0, 4, 2])
    o2, _ = orc.attend(q, k2, v, sel, np.zeros(1, np.int32), np.array([43]), 0.088)
    for h in range(16):
        g = h // 4
        toks = list(range(0, 8)) + list(range(32, 40)) + list(range(16, 24)) + list(range(40, 44))
        assert np.allclose(o2[0, h], vf[0, toks, g].mean(0), rtol=1e-12, atol=1e-12)


def test_attend_rejects_noncausal_selection(orc):
    q, k, v = _attn_inputs(5, 1, 64, 1)
    sel = np.full((1, 4, 4), -1, np.int32)
    sel[0, 0, 0] = 5                              # region 5 is the row's own (p = 43)
    with pytest.raises(ValueError):
        orc.attend(q, k, v, sel, np.zeros(1, np.int32), np.array([43]), 0.1)


# ---- fused projection [vLLM Step5FusedQKVIndexerLinear] -----------------------
# One product hidden @ W^T with the weight's rows ordered [q | k | v |
# index_q | index_k | index_z | gate], split by column ranges.


def test_project_one_hot_weights_pick_hidden_columns(orc):
    """W[n] one-hot at column perm[n]: out[r, n] is hidden[r, perm[n]]
    exactly (catches a transposed operand or a wrong row or column)."""
    rng = np.random.default_rng(3)
    H, N = 96, 150
    h = _bf(rng.standard_normal((5, H)))
    perm = rng.integers(0, H, N)
    perm[:3] = [0, H - 1, H // 2]
    w = np.zeros((N, H), np.float32)
    w[np.arange(N), perm] = 1.0
    out, _ = orc.project(h, _bf(w), (N, 0, 0, 0, 0, 0, 0))
    assert np.array_equal(out, _f(h).astype(np.float64)[:, perm])


def test_project_rank_one_closed_form(orc):
    """W = u v^T with small integers: out[r, n] = u[n] (hidden[r] . v),
    exact in fp64 (every product and partial sum is a small integer)."""
    rng = np.random.default_rng(5)
    H, N = 200, 70
    h = rng.integers(-8, 9, (4, H)).astype(np.float32)
    u = rng.integers(-5, 6, N).astype(np.float32)
    v = rng.integers(-5, 6, H).astype(np.float32)
    out, _ = orc.project(_bf(h), _bf(np.outer(u, v)), (30, 10, 10, 10, 5, 4, 1))
    assert np.array_equal(out, np.outer(h.astype(np.float64) @ v, u))


def test_project_linear_in_hidden(orc):
    rng = np.random.default_rng(7)
    H, N = 64, 40
    h1 = rng.integers(-16, 17, (3, H)).astype(np.float32)
    h2 = rng.integers(-16, 17, (3, H)).astype(np.float32)
    w = _bf(rng.integers(-4, 5, (N, H)).astype(np.float32))
    sizes = (N, 0, 0, 0, 0, 0, 0)
    a, _ = orc.project(_bf(h1), w, sizes)
    b, _ = orc.project(_bf(h2), w, sizes)
    c, _ = orc.project(_bf(h1 + h2), w, sizes)
    assert np.array_equal(c, a + b)


def test_project_split_follows_the_weight_row_order(orc):
    """The layer's geometry (16 q heads x 128, 4 KV heads x 128, indexer
    16 x 64 q and 4 x 64 k and z, a 16-column gate): weight row n holds the
    binary digits of n, hidden the powers of two, so out[:, n] = n and each
    part is its column range: q 0.., k 2048.., v 2560.., index_q 3072..,
    index_k 4096.., index_z 4352.., gate 4608..4623."""
    sizes = orc.proj_sizes()
    assert sizes == (2048, 512, 512, 1024, 256, 256, 16)
    N, H = sum(sizes), 16
    n = np.arange(N)
    w = ((n[:, None] >> np.arange(H)[None, :]) & 1).astype(np.float32)
    h = np.tile((2.0 ** np.arange(H)).astype(np.float32), (2, 1))
    out, parts = orc.project(_bf(h), _bf(w), sizes)
    assert np.array_equal(out[0], n.astype(np.float64))
    starts = dict(q=0, k=2048, v=2560, index_q=3072, index_k=4096, index_z=4352, gate=4608)
    for name, size in zip(orc.PROJ_PARTS, sizes):
        assert parts[name].shape == (2, size)
        assert np.array_equal(parts[name][1], starts[name] + np.arange(size, dtype=np.float64))
