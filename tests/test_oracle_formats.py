"""Pins of the oracle's number formats and its exp, against definitions that do
not run through the oracle: exact arithmetic in Python, torch's own casts,
the OCP E4M3 value table, and fp64 exp.

The e4m3 route "rounded through bf16 to e4m3" is the one the TensorFold
Step-5 page (pull request #903, indexer commit note) states for summaries.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- bf16 ----------------------------------------------------------------

def _bf16_nearest_even(bits32: np.ndarray) -> np.ndarray:
    """Independent fp32 -> bf16 RNE: pick the nearer of the two bf16 neighbours
    by exact float64 distance; ties go to the even pattern."""
    lo = (bits32 & 0xFFFF0000).astype(np.uint32)
    hi = lo + 0x10000
    x = bits32.view(np.float32).astype(np.float64)
    vlo = lo.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        vhi = hi.view(np.float32).astype(np.float64)
    dlo = np.abs(x - vlo)
    dhi = np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (((lo >> 16) & 1) == 1))
    return np.where(pick_hi, hi >> 16, lo >> 16).astype(np.uint16)


def test_bf16_rounding_matches_exact_nearest_even(orc):
    rng = np.random.default_rng(17)
    hi = rng.integers(0, 0x7F7F, size=200_000, dtype=np.uint32) << 16   # finite, no overflow
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    b = np.concatenate([hi[:, None] | lows[None, :], hi[:, None] | rng.integers(0, 0x10000, (hi.size, 2), dtype=np.uint32)], axis=1).ravel()
    b = np.concatenate([b, b | 0x80000000])
    got = orc.f32_to_bf16(b.view(np.float32))
    want = _bf16_nearest_even(b)
    assert np.array_equal(got, want)
    # and torch's CPU cast (round to nearest even) agrees
    t = torch.from_numpy(b.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, t)


# ---- e4m3 ----------------------------------------------------------------

def _e4m3_table():
    """Value of every finite OCP E4M3 code, from the format's definition."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = Fraction(m, 8) * Fraction(2) ** (-6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_e4m3_decode_matches_definition(orc):
    tab = _e4m3_table()
    got = orc.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    for c, v in tab.items():
        assert got[c] == float(v), hex(c)
    assert math.isnan(got[0x7F]) and math.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_from_bf16_exhaustive_brute_nearest(orc):
    """All 65,536 bf16 patterns: nearest finite code by exact rational
    distance, ties to the even code; magnitudes >= 448 saturate."""
    tab = _e4m3_table()
    pos = sorted((v, c) for c, v in tab.items() if c < 0x80)
    vals = [v for v, _ in pos]
    codes = [c for _, c in pos]
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_e4m3(h)
    f = (h.astype(np.uint32) << 16).view(np.float32)
    for i in range(65536):
        x = float(f[i])
        if not math.isfinite(x):
            continue
        a = Fraction(abs(x))
        sign = 0x80 if (h[i] & 0x8000) else 0
        if a >= 448:
            want = 0x7E | sign
        else:
            # bisect
            lo, hi = 0, len(vals) - 1
            while lo < hi:
                mid = (lo + hi + 1) // 2
                if vals[mid] <= a:
                    lo = mid
                else:
                    hi = mid - 1
            if vals[lo] == a:
                c = codes[lo]
            else:
                d0, d1 = a - vals[lo], vals[lo + 1] - a
                c = codes[lo] if d0 < d1 else codes[lo + 1] if d1 < d0 else (codes[lo] if codes[lo] % 2 == 0 else codes[lo + 1])
            want = c | sign
        assert got[i] == want, (hex(int(h[i])), x, hex(int(got[i])), hex(want))


def test_e4m3_from_bf16_matches_torch_cast(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (h.astype(np.uint32) << 16).view(np.float32)
    ok = np.isfinite(f) & (np.abs(f) < 448.0)
    t = torch.from_numpy(f[ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.bf16_to_e4m3(h[ok]), t)


def test_e4m3_golden_points(orc):
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        bits = np.array([case["bf16"]], np.uint16)
        assert int(orc.bf16_to_e4m3(bits)[0]) == case["e4m3"], case


# ---- exp -----------------------------------------------------------------

def _ulp_err(got32: np.ndarray, x32: np.ndarray) -> np.ndarray:
    ref = np.exp(x32.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    return np.abs(got32.astype(np.float64) - ref) / ulp


def test_exp_accuracy_dense_sweep(orc):
    # every 97th fp32 value in [-87, 0] (about 11 million arguments) plus a
    # dense sweep near 0 and the reduction boundaries n*ln2/2
    hi = np.float32(-87.0).view(np.uint32)
    neg = (np.arange(0x80000000, int(hi) + 1, 97, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    ks = np.arange(-126, 1, dtype=np.float64)
    edges = (ks * math.log(2) / 2).astype(np.float32)
    edge_nb = (edges.view(np.uint32)[:, None] + np.arange(-64, 65, dtype=np.int64)[None, :].astype(np.uint32)).view(np.float32).ravel()
    x = np.concatenate([neg, edge_nb[(edge_nb <= 0) & (edge_nb >= -87)], np.linspace(-1e-3, 0, 10001, dtype=np.float32)])
    got = orc.exp(x)
    err = _ulp_err(got, x)
    assert err.max() <= 1.0, (float(err.max()), float(x[np.argmax(err)]))


def test_exp_special_values_and_monotone(orc):
    assert orc.exp(np.array([0.0], np.float32))[0] == 1.0
    assert orc.exp(np.array([-0.0], np.float32))[0] == 1.0
    assert orc.exp(np.array([-200.0], np.float32))[0] == orc.exp(np.array([-87.0], np.float32))[0]
    v = orc.exp(np.array([-87.0], np.float32))[0]
    assert v >= np.finfo(np.float32).tiny            # never subnormal
    x = np.sort(np.random.default_rng(41).uniform(-87, 0, 2_000_000).astype(np.float32))
    y = orc.exp(x)
    assert np.all(np.diff(y) >= 0)
    assert orc.exp(np.array([-math.log(2)], np.float32))[0] == pytest.approx(0.5, rel=1.2e-7)


def test_exp_bits_range_is_exp_of_those_inputs(orc):
    """The range sweep helper (used to check the GPU's exp over whole ranges
    of bit patterns) evaluates the same exp as exp() on an input array."""
    for start, n in ((0x80000000, 5000), (0xC2AD0000, 70000), (0x3F800000 - 100, 300)):
        x = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = orc.exp(x)
        got = orc.exp_bits_range(start, n)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
