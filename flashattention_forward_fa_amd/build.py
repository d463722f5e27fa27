"""Build libfa.so in-tree with hipcc for gfx950.

The library is one shared object holding the C ABI (``csrc/fa_api.cpp``) and
the HIP kernels (``csrc/fa_fwd_kernel.hip``, ``csrc/fa_bwd_kernel.hip``).  Packed-fp32 VALU
instructions are disabled for device code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
SOURCES = [os.path.join(CSRC, "fa_fwd_kernel.hip"), os.path.join(CSRC, "fa_bwd_kernel.hip"),
           os.path.join(CSRC, "fa_clock.hip"), os.path.join(CSRC, "fa_api.cpp")]
ARCH = "gfx950"

# -amdgpu-mfma-vgpr-form: MFMA results and accumulators in ordinary VGPRs.  The
# backward kernels hold more accumulators than the compiler's AGPR heuristic
# expects and otherwise get register-file copies of them every block; the
# forward kernel's code is the same either way.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


LIB_TRACE = os.path.join(HERE, "libfa_trace.so")


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile every source into libfa.so (always recompiles); trace=True builds
    the timeline flavour libfa_trace.so instead (FA_TRACE: the forward kernel
    records shader-clock stamps at its phase boundaries into opts.trace)."""
    lib = LIB_TRACE if trace else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DFA_TRACE"] if trace else []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # Resolve every symbol now: a kernel whose launch stub the host pass did
    # not emit would otherwise only fail when the library is loaded.
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
