"""The gfx950 builds of the summary kernel's helpers: the hardware
conversions (bf16 and e4m3 rounding by gfx950's conversion instructions)
against the software forms over every input, the software forms being pinned
to the oracle on the CPU (test_device_helpers_host.py); and the fixed exp,
compiled for gfx950, against the oracle's exp bit for bit over every fp32 of
the summary's domain [-87, 0], the clamp edges and the positive side."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "_device_check.so")

pytestmark = pytest.mark.gpu


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build()")
    L = C.CDLL(LIB)
    for f in (L.device_check_bf16, L.device_check_e4m3):
        f.restype = C.c_int
        f.argtypes = [C.c_void_p, C.c_void_p]
    return L


@pytest.mark.parametrize("name", ["bf16", "e4m3"])
def test_hardware_conversion_matches_software_everywhere(name):
    L = _lib()
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")  # 0xffffffff
    fn = L.device_check_bf16 if name == "bf16" else L.device_check_e4m3
    assert fn(C.c_void_p(bad.data_ptr()), C.c_void_p(first.data_ptr())) == 0
    n = int(bad.item())
    assert n == 0, f"{name}: {n} mismatches, first input 0x{int(first.item()) & 0xffffffff:08x}"


def _exp_lib():
    L = _lib()
    L.device_exp_range.restype = C.c_int
    L.device_exp_range.argtypes = [C.c_uint32, C.c_uint32, C.c_void_p]
    L.device_exp_list.restype = C.c_int
    L.device_exp_list.argtypes = [C.c_void_p, C.c_void_p, C.c_uint32]
    return L


def _check_exp_bits(orc, x, got, where, want=None):
    want = orc.exp(x) if want is None else want
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    if bad.size:
        xb = x[bad[0]] if x is not None else "?"
        raise AssertionError(f"{where}: {bad.size} mismatches, first at {bad[0]} x={xb!r} "
                             f"gpu={got[bad[0]]!r} oracle={want[bad[0]]!r}")


def test_exp_fixed_gfx950_every_fp32_in_summary_domain(orc):
    """Every fp32 bit pattern from -0 down to -87 (the clamp), 1.1e9 inputs, in
    chunks of 2^26: the GPU's exp_fixed equals the oracle's exp bit for bit."""
    L = _exp_lib()
    lo = 0x80000000                                              # -0.0
    hi = int(np.array([-87.0], np.float32).view(np.uint32)[0])   # -87.0, inclusive
    chunk = 1 << 26
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    n_done = 0
    for start in range(lo, hi + 1, chunk):
        n = min(chunk, hi + 1 - start)
        assert L.device_exp_range(start, n, C.c_void_p(out.data_ptr())) == 0
        got = out[:n].cpu().numpy()
        want = orc.exp_bits_range(start, n)
        if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
            x = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
            _check_exp_bits(orc, x, got, f"bits 0x{start:08x}+{n}", want)
        n_done += n
    assert n_done == hi + 1 - lo


def test_exp_fixed_gfx950_clamp_edges_and_positive_side(orc):
    """Below the clamp (-87 .. -200 and -inf), the positive side up to and past
    the upper clamp (88), zeros, subnormals: bit-exact against the oracle."""
    L = _exp_lib()
    below = np.arange(int(np.array([-87.0], np.float32).view(np.uint32)[0]),
                      int(np.array([-89.0], np.float32).view(np.uint32)[0]) + 1,
                      dtype=np.uint64).astype(np.uint32).view(np.float32)
    pos = np.arange(0, int(np.array([90.0], np.float32).view(np.uint32)[0]), 7,
                    dtype=np.uint64).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 88.0, 88.5, -200.0, 200.0,
                        np.float32(-87.0), np.nextafter(np.float32(-87.0), np.float32(0))],
                       np.float32)
    x = np.concatenate([below, pos, special]).astype(np.float32)
    xd = torch.from_numpy(x).to("cuda")
    out = torch.empty_like(xd)
    assert L.device_exp_list(C.c_void_p(xd.data_ptr()), C.c_void_p(out.data_ptr()), x.size) == 0
    _check_exp_bits(orc, x, out.cpu().numpy(), "edges")
