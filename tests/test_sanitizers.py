"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* ``oracle/oracle.c`` built with gcc ``-fsanitize=address,undefined`` runs
  every pin of ``tests/oracle_pins.py`` in a child process with gcc's ASan
  runtime preloaded.
* The C ABI's host code (``csrc/fa_api.cpp``) built with clang
  ``-fsanitize=address,undefined`` -- with stand-ins for the four kernel
  launchers, since no argument check ever reaches a launch and device code is
  not instrumented -- runs ``tests/test_abi.py`` in a child process with
  clang's ASan runtime preloaded.
* Each build is first shown to report a planted mistake (an out-of-bounds read
  in a copy of the oracle, a signed overflow in a copy of fa_api.cpp), so that
  a clean run means something.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
CSRC = os.path.join(ROOT, "flashattention_forward_fa_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "OMP_NUM_THREADS": "4"}
REPORTS = ("ERROR: AddressSanitizer", "runtime error:")


def _runtime(compiler, name):
    """Path of a sanitizer runtime as the compiler resolves it, or None."""
    try:
        out = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True,
                             text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _child(code, preload, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


# ----------------------------------------------------------------- the oracle

def _build_oracle(src, out):
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-fopenmp",
                    "-fPIC", "-shared", "-std=c11", "-o", str(out), str(src), "-lm"], check=True)


_PINS = """
import sys
from oracle import Oracle
from tests import oracle_pins
orc = Oracle({lib!r})
for pin in oracle_pins.{pins}:
    pin(orc)
print("PINS DONE", flush=True)
"""


@pytest.fixture(scope="module")
def gcc_asan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    rt = _runtime("gcc", "libasan.so")
    if rt is None:
        pytest.skip("gcc's ASan runtime not found")
    return rt


def test_oracle_sanitizer_build_reports_a_planted_overflow(tmp_path, gcc_asan):
    src = open(ORACLE_C).read()
    # Every dot product reads one element past its key row: past the end of
    # K on the last key.
    old = "for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];"
    assert src.count(old) == 1
    (tmp_path / "bad.c").write_text(src.replace(old, old.replace("c < d", "c <= d")))
    _build_oracle(tmp_path / "bad.c", tmp_path / "libbad.so")
    r = _child(_PINS.format(lib=str(tmp_path / "libbad.so"), pins="ALL_PINS[:1]"), gcc_asan)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_under_sanitizers(tmp_path, gcc_asan):
    _build_oracle(ORACLE_C, tmp_path / "liboracle_san.so")
    r = _child(_PINS.format(lib=str(tmp_path / "liboracle_san.so"), pins="ALL_PINS"), gcc_asan)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "PINS DONE" in r.stdout
    assert not any(s in r.stderr for s in REPORTS), r.stderr[-4000:]


# ----------------------------------------------------- the library's host code

# Stand-ins for the kernel launchers (fa_internal.h): every check returns
# before a launch, and a launch that were reached would report a HIP error.
_STUBS = """
#include <stdint.h>
#include "fa_internal.h"
FA_NS_BEGIN
int launch_fwd(const FwdParams &, int, bool, OutType, void *) { return 100; }
int launch_bwd(const BwdParams &, int, bool, void *) { return 100; }
int bwd_scratch(void **ptr) { *ptr = nullptr; return -1; }
int launch_clock_probe(uint64_t *, int, unsigned, void *) { return 100; }
FA_NS_END
"""

_ABI = """
import sys
import flashattention_forward_fa_amd as fa
fa.library_path = lambda: {lib!r}
import pytest
# -s: a sanitizer report goes to this process's stderr, not into pytest's capture
sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu", {sel!r}]))
"""


@pytest.fixture(scope="module")
def clang_asan():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    rt = _runtime(CLANG, "libclang_rt.asan-x86_64.so")
    if rt is None:
        pytest.skip("clang's ASan runtime not found")
    return rt


def _build_host(api_src, tmp_path, name):
    stubs = tmp_path / "stubs.cpp"
    stubs.write_text(_STUBS)
    out = tmp_path / name
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                    str(api_src), str(stubs), f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", str(out)], check=True)
    return out


def test_host_sanitizer_build_reports_a_planted_overflow(tmp_path, clang_asan):
    src = open(os.path.join(CSRC, "fa_api.cpp")).read()
    # The tile count multiplied in 32 bits: overflows for the sizes that the
    # size check exists to reject.
    old = "if ((int64_t)B * H * num_m >= (int64_t)1 << 31) return FA_ERR_INVALID_ARG;"
    assert src.count(old) == 1
    bad = tmp_path / "fa_api.cpp"
    bad.write_text(src.replace(old, old.replace("(int64_t)B * H * num_m", "(int64_t)(B * H * (int)num_m)")))
    lib = _build_host(bad, tmp_path, "libfa_bad.so")
    r = _child(_ABI.format(lib=str(lib), sel="tests/test_abi.py::test_size_overflow_rejected"),
               clang_asan)
    assert r.returncode != 0
    assert "signed integer overflow" in r.stderr, r.stderr[-2000:]


def test_host_code_under_sanitizers(tmp_path, clang_asan):
    lib = _build_host(os.path.join(CSRC, "fa_api.cpp"), tmp_path, "libfa_san.so")
    r = _child(_ABI.format(lib=str(lib), sel="tests/test_abi.py"), clang_asan)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
    assert not any(s in r.stderr for s in REPORTS), r.stderr[-4000:]
