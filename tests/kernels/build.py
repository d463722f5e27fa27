"""Build tests/kernels/libfa_unit.so (test-only kernels over the library's
device helpers) with the flags the library itself is built with."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
LIB = os.path.join(HERE, "libfa_unit.so")


def build() -> str:
    from flashattention_forward_fa_amd import build as fa_build
    tmp = LIB + ".tmp"
    subprocess.run([fa_build.hipcc(), *fa_build.HIPCC_FLAGS, os.path.join(HERE, "fa_unit.hip"),
                    "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
