"""The hardware conversions used by the summary kernel (bf16 and e4m3
rounding by gfx950's conversion instructions) against the software forms
over every input; the software forms are pinned to the oracle on the CPU
(test_device_helpers_host.py)."""
import ctypes as C
import os

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
