"""The C-ABI library: it loads, exports every function include/fa.h declares,
and its argument checks return the documented status codes (no GPU: the checks
run before any HIP call)."""
import ctypes
import math
import os
import re

import pytest

import flashattention_forward_fa_amd as fa


def _read(path):
    with open(path) as f:
        return f.read()


HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")
P = 1 << 20          # a 16-byte aligned stand-in address; the checks never dereference it


def declared_functions():
    text = _read(HEADER)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = ctypes.CDLL(fa.library_path())
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_ex", "fa_fwd_check", "fa_status_string",
            "fa_fwd_opts_default", "fa_version", "fa_bwd", "fa_bwd_check",
            "fa_bwd_workspace_size"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_defaults():
    assert fa.fa_version() >= 100
    o = fa.fa_fwd_opts_default()
    assert (o.o_dtype, o.rescale_threshold, o.schedule, o.kv_heads) == (0, 8.0, 0, 0)
    assert o.rescale_counts is None   # NULL: no counting


def test_rescale_counts_pointer():
    assert check(opts=opts(rescale_counts=P)) == fa.FA_OK
    assert check(opts=opts(rescale_counts=P + 2)) == fa.FA_ERR_INVALID_ARG   # 4-byte aligned
    assert check(opts=opts(rescale_counts=P + 4)) == fa.FA_OK


def test_status_strings():
    assert fa.fa_status_string(fa.FA_OK) == "ok"
    assert "invalid" in fa.fa_status_string(fa.FA_ERR_INVALID_ARG)
    assert "unsupported" in fa.fa_status_string(fa.FA_ERR_UNSUPPORTED)
    assert "HIP" in fa.fa_status_string(fa.FA_ERR_HIP)
    assert fa.fa_status_string(12345) == "unknown status"


def check(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, Nq=100, Nk=100, d=128, scale=0.1, causal=1,
             varlen_offsets=None, opts=None)
    a.update(kw)
    return fa.fa_fwd_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                           a["Nk"], a["d"], a["scale"], a["causal"], a["varlen_offsets"], a["opts"])


def opts(**kw):
    o = fa.fa_fwd_opts_default()
    for key, val in kw.items():
        setattr(o, key, val)
    return o


def test_valid_arguments():
    assert check() == fa.FA_OK
    assert check(d=64, causal=0) == fa.FA_OK
    assert check(varlen_offsets=P, Nq=8192, Nk=8192) == fa.FA_OK
    assert check(scale=-0.5) == fa.FA_OK and check(scale=0.0) == fa.FA_OK
    assert check(opts=opts(o_dtype=fa.FA_DTYPE_F32, rescale_threshold=0.0,
                           schedule=fa.FA_SCHEDULE_LPT)) == fa.FA_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_and_misaligned_pointers(field):
    assert check(**{field: None}) == fa.FA_ERR_INVALID_ARG
    assert check(**{field: P + 8}) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [("B", 0), ("H", 0), ("Nq", 0), ("Nk", -3), ("d", 0),
                                         ("causal", 2), ("scale", math.inf),
                                         ("scale", math.nan)])
def test_bad_sizes(field, value):
    assert check(**{field: value}) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [32, 80, 96, 192, 256])
def test_unsupported_head_dim(d):
    assert check(d=d) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("tau", [-1.0, 64.5, math.inf, math.nan])
def test_bad_threshold(tau):
    assert check(opts=opts(rescale_threshold=tau)) == fa.FA_ERR_INVALID_ARG


def test_bad_options():
    assert check(opts=opts(o_dtype=7)) == fa.FA_ERR_UNSUPPORTED
    assert check(opts=opts(schedule=3)) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("H,kv,status", [(8, 0, 0), (8, 8, 0), (8, 4, 0), (8, 2, 0), (8, 1, 0),
                                         (8, 3, -1), (8, 16, -1), (8, -1, -1), (6, 4, -1),
                                         (6, 3, 0)])
def test_kv_heads(H, kv, status):
    """Grouped K/V heads: 0 (= H) or a divisor of H."""
    assert check(H=H, opts=opts(kv_heads=kv)) == status


def test_varlen_rules():
    assert check(varlen_offsets=P, Nq=100, Nk=200) == fa.FA_ERR_INVALID_ARG
    assert check(varlen_offsets=P + 2, Nq=100, Nk=100) == fa.FA_ERR_INVALID_ARG


def test_size_overflow_rejected():
    assert check(B=1 << 20, H=1 << 10, Nq=1 << 16, Nk=16) == fa.FA_ERR_INVALID_ARG
    # a 256-row tile's byte offsets must fit 32 bits: H*d < 2^23
    assert check(H=1 << 16, d=128) == fa.FA_ERR_INVALID_ARG
    assert check(H=(1 << 16) - 1, d=128) == fa.FA_OK


def test_rejected_launch_makes_no_hip_call():
    """fa_fwd with a bad argument returns before touching HIP (safe without a GPU)."""
    st = fa.fa_fwd(None, P, P, P, P, 1, 1, 16, 16, 128, 0.1, 0, None, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_fwd(P, P, P, P, P, 1, 1, 16, 16, 96, 0.1, 0, None, stream=0)
    assert st == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ backward entry points

def bcheck(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, ws=P, B=2, H=4, Nq=100, Nk=100,
             d=128, scale=0.1, causal=1, varlen_offsets=None, kv_heads=0)
    a.update(kw)
    return fa.fa_bwd_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                           a["dv"], a["ws"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                           a["causal"], a["varlen_offsets"], a["kv_heads"])


def test_bwd_valid_arguments():
    assert bcheck() == fa.FA_OK
    assert bcheck(d=64, causal=0, kv_heads=2) == fa.FA_OK
    assert bcheck(varlen_offsets=P, Nq=512, Nk=512) == fa.FA_OK
    assert bcheck(scale=-1.0) == fa.FA_OK and bcheck(scale=0.0) == fa.FA_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"])
def test_bwd_null_pointer(field):
    assert bcheck(**{field: None}) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["dout", "dq", "dk", "dv"])
def test_bwd_misaligned(field):
    assert bcheck(**{field: P + 8}) == fa.FA_ERR_INVALID_ARG


def test_bwd_rules():
    assert bcheck(ws=P + 2) == fa.FA_ERR_INVALID_ARG          # workspace: 4-byte aligned
    assert bcheck(ws=P + 4) == fa.FA_OK
    assert bcheck(kv_heads=3) == fa.FA_ERR_INVALID_ARG         # must divide H
    assert bcheck(d=96) == fa.FA_ERR_UNSUPPORTED
    assert bcheck(causal=2) == fa.FA_ERR_INVALID_ARG
    assert bcheck(scale=math.nan) == fa.FA_ERR_INVALID_ARG
    assert bcheck(varlen_offsets=P, Nq=100, Nk=200) == fa.FA_ERR_INVALID_ARG


def test_bwd_workspace_size():
    assert fa.fa_bwd_workspace_size(2, 4, 100) == 4 * 2 * 4 * 100
    assert fa.fa_bwd_workspace_size(0, 4, 100) == 0


def test_bwd_rejected_launch_makes_no_hip_call():
    st = fa.fa_bwd(P, P, P, P, P, None, P, P, P, P, 1, 1, 16, 16, 128, 0.1, 0, None, 0, stream=0)
    assert st == fa.FA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    """The Python wrappers refuse tensors that are not on the GPU before loading
    the library or launching anything (a host pointer would be dereferenced on
    the device)."""
    import torch
    q = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.attention(q, q, q, 0.125, True)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.flash_attention(q, q, q, 0.125, True)
    lse = torch.zeros((1, 2, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.attention_bwd(q, q, q, q, lse, q, 0.125, True)
    packed = torch.zeros((8, 2, 64), dtype=torch.bfloat16)
    off = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.attention(packed, packed, packed, 0.125, True, varlen_offsets=off, max_seqlen=8)


def test_clock_probe_argument_checks():
    """fa_clock_probe rejects bad arguments before any HIP call."""
    lib = fa.load()
    ref = ctypes.c_double(0.0)
    bad = [(0, 10, 10, ctypes.byref(ref)),          # null samples
           (P + 4, 10, 10, ctypes.byref(ref)),      # not 8-byte aligned
           (P, 1, 10, ctypes.byref(ref)),           # fewer than two samples
           (P, 1000001, 10, ctypes.byref(ref)),
           (P, 10, 0, ctypes.byref(ref)),           # interval out of range
           (P, 10, 100001, ctypes.byref(ref)),
           (P, 10, 10, None)]                        # no place for the rate
    for samples, n, us, out in bad:
        assert lib.fa_clock_probe(samples or None, n, us, out, None) == fa.FA_ERR_INVALID_ARG


def test_noalloc_checks_without_a_gpu():
    """fa_bwd_noalloc_check: the fa_bwd checks without a workspace argument, plus
    the size bound of the static array (FA_ERR_TOO_LARGE), no HIP call."""
    lib = fa.load()
    cap = fa.fa_bwd_noalloc_max_bytes()
    assert cap == 32 << 20
    H, d = 32, 128
    fits = cap // (4 * H)                      # 4 * H * Nq == cap
    args = lambda Nq: (P,) * 9 + (1, H, Nq, Nq, d, 0.1, 1, None, 0)
    assert fa.fa_bwd_noalloc_check(*args(fits)) == fa.FA_OK
    assert fa.fa_bwd_noalloc_check(*args(fits + 1)) == fa.FA_ERR_TOO_LARGE
    assert "scratch" in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)
    bad = (P,) * 8 + (0,) + (1, H, 100, 100, d, 0.1, 1, None, 0)   # null dv
    assert fa.fa_bwd_noalloc_check(*bad) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_noalloc_check is not None


def test_library_binds_after_torch():
    """Loading the library imports torch first, so libfa resolves the HIP
    runtime torch already loaded instead of a second copy (checked here from
    the process's mapped libraries: exactly one libamdhip64 after load)."""
    import subprocess
    import sys
    code = ("import flashattention_forward_fa_amd as fa; fa.load(); "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_exp2_poly_option_checks():
    """exp2_poly: 0, 4, 8 or 16; nonzero needs tau <= 15 (fp16 P), bf16 O and no
    rescale counts."""
    P = 1 << 20
    opts = fa.fa_fwd_opts_default()
    assert opts.exp2_poly == 0
    chk = lambda o: fa.fa_fwd_check(P, P, P, P, P, 1, 2, 64, 64, 128, 0.1, 1, None, o)
    opts.exp2_poly = 8
    assert chk(opts) == fa.FA_OK
    for good in (4, 16):
        opts.exp2_poly = good
        assert chk(opts) == fa.FA_OK
    for bad in (2, 12, 32, -1):
        opts.exp2_poly = bad
        assert chk(opts) == fa.FA_ERR_UNSUPPORTED
    opts.exp2_poly = 8
    opts.o_dtype = fa.FA_DTYPE_F32
    assert chk(opts) == fa.FA_ERR_UNSUPPORTED
    opts.o_dtype = fa.FA_DTYPE_BF16
    opts.exp2_poly = 8
    opts.rescale_threshold = 20.0
    assert chk(opts) == fa.FA_ERR_UNSUPPORTED
    opts.rescale_threshold = 8.0
    opts.rescale_counts = P
    assert chk(opts) == fa.FA_ERR_UNSUPPORTED
