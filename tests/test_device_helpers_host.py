"""The GPU path's format and exp helpers (csrc/device.hpp), compiled for the
host, agree bit for bit with the oracle's independent implementations: every
bf16 pattern to e4m3, fp32 to bf16 rounding, and the fixed exp over a dense
sweep of its domain. A logic slip in the device code shows here, on the CPU,
before any GPU run; the GPU parity tests then cover the gfx950 build."""
import ctypes as C
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_helpers.hip")
HDR = os.path.join(ROOT, "long_context_sparse_indexer_amd", "csrc", "device.hpp")
LIB = os.path.join(ROOT, "_build", "libstep5_hosthelpers.so")


@pytest.fixture(scope="module")
def ht():
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(SRC), os.path.getmtime(HDR)):
        cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC",
               "-shared", "-ffp-contract=off", SRC, "-o", LIB]
        subprocess.run(cmd, check=True, capture_output=True)
    L = C.CDLL(LIB)
    P, I64 = C.c_void_p, C.c_int64
    for f in ("ht_e4m3_from_bf16", "ht_bf16_bits", "ht_exp"):
        getattr(L, f).argtypes = [P, P, I64]
    L.ht_pair8.restype = C.c_float
    L.ht_pair8.argtypes = [P]
    return L


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def test_e4m3_all_bf16_patterns(ht, orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (h.astype(np.uint32) << 16).view(np.float32)
    h = h[np.isfinite(f)]
    got = np.empty(h.shape, np.uint8)
    ht.ht_e4m3_from_bf16(_p(h), _p(got), h.size)
    assert np.array_equal(got, orc.bf16_to_e4m3(h))


def test_bf16_rounding(ht, orc):
    rng = np.random.default_rng(1)
    b = rng.integers(0, 0x7F7F0000, 2_000_000, dtype=np.uint32)
    b = np.concatenate([b, b | 0x80000000, (b & 0xFFFF0000) | 0x8000, (b & 0xFFFF0000) | 0x7FFF])
    x = b.view(np.float32)
    got = np.empty(x.shape, np.uint16)
    ht.ht_bf16_bits(_p(x), _p(got), x.size)
    assert np.array_equal(got, orc.f32_to_bf16(x))


def test_exp_matches_oracle_bitwise(ht, orc):
    hi = np.float32(-87.0).view(np.uint32)
    x = np.arange(0x80000000, int(hi) + 64, 13, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, np.linspace(-200, 100, 100001, dtype=np.float32)])
    got = np.empty(x.shape, np.float32)
    ht.ht_exp(_p(x), _p(got), x.size)
    want = orc.exp(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_pair8_matches_oracle_blocks(ht, orc):
    rng = np.random.default_rng(2)
    for _ in range(500):
        x = (rng.standard_normal(64) * np.exp(rng.uniform(-5, 5, 64))).astype(np.float32)
        blocks = np.array([ht.ht_pair8(_p(np.ascontiguousarray(x[8 * c:8 * c + 8]))) for c in range(8)],
                          np.float32)
        assert np.float32(ht.ht_pair8(_p(blocks))) == np.float32(orc.sum64(x))
