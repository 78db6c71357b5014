"""Builds tests/_device_check.so (GPU checks of the device helpers) for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
LIB = os.path.join(HERE, "_device_check.so")


def build() -> str:
    from long_context_sparse_indexer_amd import _build as b
    src = os.path.join(HERE, "device_check.hip")
    tmp = LIB + ".tmp"
    cmd = [b.hipcc(), *b.flags(), "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on device_check.hip:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
