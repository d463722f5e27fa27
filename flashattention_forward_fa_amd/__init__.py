"""MI355X-native FlashAttention forward: Python binding over the C-ABI library libfa.

The binding only marshals arguments; every step of the attention forward runs
in the HIP kernels of ``libfa.so`` (built in-tree by ``build.py``).  The
library is loaded on first use; a missing or unloadable library raises -- there
is no CPU fallback.

Entry points mirror ``include/fa.h``: ``fa_fwd``, ``fa_fwd_ex``,
``fa_fwd_check``, ``fa_status_string``, ``fa_fwd_opts_default``,
``fa_version``.  Pointer arguments accept torch tensors (their data pointer) or
integers; ``stream`` accepts a ``torch.cuda.Stream``, an integer hipStream_t or
None (torch's current stream).  ``attention`` is a convenience wrapper that
allocates O and LSE with torch and raises on a non-zero status; ``attention_bwd``
does the same for the backward, and ``flash_attention`` joins the two as one
differentiable torch operation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_TOO_LARGE",
           "FA_DTYPE_BF16", "FA_DTYPE_F32", "FA_SCHEDULE_AUTO", "FA_SCHEDULE_LINEAR",
           "FA_SCHEDULE_LPT", "FaFwdOpts", "FaError", "library_path", "load", "fa_fwd",
           "fa_fwd_ex", "fa_fwd_check", "fa_status_string", "fa_fwd_opts_default",
           "fa_version", "fa_bwd", "fa_bwd_check", "fa_bwd_workspace_size", "fa_bwd_noalloc",
           "fa_bwd_noalloc_check", "fa_bwd_noalloc_max_bytes", "fa_clock_probe",
           "attention",
           "attention_bwd", "flash_attention"]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, -1, -2, -3, -4
FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1
FA_SCHEDULE_AUTO, FA_SCHEDULE_LINEAR, FA_SCHEDULE_LPT = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str = "fa_fwd"):
        super().__init__(f"{what} returned {status} ({fa_status_string(status)})")
        self.status = status


class FaFwdOpts(ctypes.Structure):
    """Mirror of ``fa_fwd_opts`` in include/fa.h."""
    _fields_ = [("o_dtype", ctypes.c_int32), ("rescale_threshold", ctypes.c_float),
                ("schedule", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("rescale_counts", ctypes.c_void_p), ("trace", ctypes.c_void_p),
                ("trace_workgroups", ctypes.c_int32), ("exp2_poly", ctypes.c_int32)]


def _bind_torch_hip_runtime():
    """Import torch before the library is loaded.  torch brings its own HIP
    runtime and asks for it by an unversioned name; libfa asks for
    libamdhip64.so.7.  Loaded after torch, libfa binds to torch's runtime (same
    SONAME); loaded first, it would pull in the system runtime, torch would
    then load its own beside it, and launches from libfa would go to a runtime
    that does not own torch's memory and streams.  Without torch there is only
    the system runtime and nothing to do."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load():
    """Load libfa.so (once).  Raises if it is missing: build it with build.py."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libfa.so not found at {path}; build it with "
                           f"`python -m flashattention_forward_fa_amd.build`")
    _bind_torch_hip_runtime()
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    common = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.argtypes = common + [vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_ex.argtypes = common + [vp, ctypes.POINTER(FaFwdOpts)]
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_check.argtypes = common + [ctypes.POINTER(FaFwdOpts)]
    lib.fa_fwd_check.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd_opts_default.argtypes = [ctypes.POINTER(FaFwdOpts)]
    lib.fa_fwd_opts_default.restype = None
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    bwd = [vp] * 10 + [i, i, i, i, i, f, i, vp, i]
    lib.fa_bwd.argtypes = bwd + [vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_check.argtypes = bwd
    lib.fa_bwd_check.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_int64
    nb = [vp] * 9 + [i, i, i, i, i, f, i, vp, i]
    lib.fa_bwd_noalloc.argtypes = nb + [vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_check.argtypes = nb
    lib.fa_bwd_noalloc_check.restype = i
    lib.fa_bwd_noalloc_max_bytes.argtypes = []
    lib.fa_bwd_noalloc_max_bytes.restype = ctypes.c_int64
    lib.fa_clock_probe.argtypes = [vp, i, i, ctypes.POINTER(ctypes.c_double), vp]
    lib.fa_clock_probe.restype = i
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def fa_fwd_opts_default() -> FaFwdOpts:
    opts = FaFwdOpts()
    load().fa_fwd_opts_default(ctypes.byref(opts))
    return opts


def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets=None,
           stream=None) -> int:
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                         float(scale), int(causal), _ptr(varlen_offsets), _stream(stream))


def fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets=None,
              stream=None, opts: FaFwdOpts | None = None) -> int:
    return load().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                            float(scale), int(causal), _ptr(varlen_offsets), _stream(stream),
                            ctypes.byref(opts) if opts is not None else None)


def fa_fwd_check(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets=None,
                 opts: FaFwdOpts | None = None) -> int:
    return load().fa_fwd_check(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk,
                               d, float(scale), int(causal), _ptr(varlen_offsets),
                               ctypes.byref(opts) if opts is not None else None)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale, causal,
           varlen_offsets=None, kv_heads=0, stream=None) -> int:
    return load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                         _ptr(dk), _ptr(dv), _ptr(workspace), B, H, Nq, Nk, d, float(scale),
                         int(causal), _ptr(varlen_offsets), int(kv_heads), _stream(stream))


def fa_bwd_check(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale, causal,
                 varlen_offsets=None, kv_heads=0) -> int:
    return load().fa_bwd_check(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), B, H, Nq, Nk, d,
                               float(scale), int(causal), _ptr(varlen_offsets), int(kv_heads))


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal,
                   varlen_offsets=None, kv_heads=0, stream=None) -> int:
    return load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, float(scale),
                                 int(causal), _ptr(varlen_offsets), int(kv_heads), _stream(stream))


def fa_bwd_noalloc_check(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale, causal,
                         varlen_offsets=None, kv_heads=0) -> int:
    return load().fa_bwd_noalloc_check(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                       _ptr(dq), _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, float(scale),
                                       int(causal), _ptr(varlen_offsets), int(kv_heads))


def fa_bwd_noalloc_max_bytes() -> int:
    return int(load().fa_bwd_noalloc_max_bytes())


def fa_bwd_workspace_size(B: int, H: int, Nq: int) -> int:
    return int(load().fa_bwd_workspace_size(B, H, Nq))


def fa_clock_probe(samples, n: int, interval_us: int, stream=None):
    """Launch the shader-clock probe (diagnostics); returns (status, ref_hz).
    samples: device buffer of 2*n uint64 (e.g. an int64 tensor)."""
    ref = ctypes.c_double(0.0)
    st = load().fa_clock_probe(_ptr(samples), int(n), int(interval_us), ctypes.byref(ref),
                               _stream(stream))
    return st, ref.value


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_version() -> int:
    return load().fa_version()


def _same_gpu(**tensors):
    """Raise ValueError unless every given tensor (None entries skipped) lives on
    one GPU: a host pointer handed to a kernel would be dereferenced on the
    device.  Runs before the library is loaded or anything is launched."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{name} must be a GPU tensor (got device {getattr(t, 'device', '?')})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    if dev is not None:
        import torch
        if dev.index is not None and dev.index != torch.cuda.current_device():
            raise ValueError(f"the tensors are on {dev}, the current device is "
                             f"cuda:{torch.cuda.current_device()}: launches go to the current device")


def attention(q, k, v, scale: float, causal: bool, *, varlen_offsets=None, max_seqlen=None,
              o_dtype=FA_DTYPE_BF16, rescale_threshold: float = 8.0,
              schedule: int = FA_SCHEDULE_AUTO, stream=None, rescale_counts: bool = False,
              exp2_poly: int = 0):
    """Allocate O and LSE with torch on q's device and run fa_fwd_ex.

    Fixed length: q [B,Nq,H,d], k/v [B,Nk,Hkv,d] bf16 -> o [B,Nq,H,d], lse [B,H,Nq].
    Varlen: q [T,H,d], k/v [T,Hkv,d] and int32 offsets [B+1] on the device,
    max_seqlen = the longest sequence -> o [T,H,d], lse [H,T].
    Hkv (read from k's shape) divides H; query heads h*G .. h*G+G-1, G = H/Hkv,
    share K/V head h.  rescale_counts=True also returns each row's count of
    rescale events (int32, laid out like lse): (o, lse, counts).
    q, k, v and the offsets must be on one GPU (ValueError otherwise).
    max_seqlen must be at least every sequence's length: the tile grid is sized
    from it, and rows of a longer sequence would be left unwritten.
    """
    import torch
    _same_gpu(q=q, k=k, v=v, varlen_offsets=varlen_offsets)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    odt = torch.float32 if o_dtype == FA_DTYPE_F32 else torch.bfloat16
    o = torch.empty(q.shape, dtype=odt, device=q.device)
    if varlen_offsets is None:
        B, Nq, H, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        if k.shape != (B, Nk, Hkv, d) or v.shape != k.shape or Hkv < 1 or H % Hkv:
            raise ValueError("k, v must be [B, Nk, Hkv, d] matching q, with Hkv dividing H")
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        T, H, d = q.shape
        Hkv = k.shape[1]
        if k.shape != (T, Hkv, d) or v.shape != k.shape or Hkv < 1 or H % Hkv:
            raise ValueError("packed k, v must be [T, Hkv, d] matching q, with Hkv dividing H")
        if varlen_offsets.dtype != torch.int32:
            raise TypeError("varlen offsets must be int32")
        B = varlen_offsets.numel() - 1
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with varlen offsets")
        Nq = Nk = int(max_seqlen)
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    opts = fa_fwd_opts_default()
    opts.o_dtype = o_dtype
    opts.rescale_threshold = rescale_threshold
    opts.schedule = schedule
    opts.kv_heads = Hkv
    opts.exp2_poly = exp2_poly
    counts = None
    if rescale_counts:
        counts = torch.zeros(lse.shape, dtype=torch.int32, device=q.device)
        opts.rescale_counts = counts.data_ptr()
    st = fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets, stream, opts)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_ex")
    return (o, lse, counts) if rescale_counts else (o, lse)


def attention_bwd(q, k, v, o, lse, dout, scale: float, causal: bool, *, varlen_offsets=None,
                  max_seqlen=None, stream=None):
    """Allocate dQ, dK, dV and the workspace with torch and run fa_bwd.

    Shapes and layouts as for attention(); o and lse are the forward's outputs
    (o bf16) and dout is dO, shaped like o.  Returns (dq, dk, dv), bf16.
    Every tensor must be on one GPU (ValueError otherwise); max_seqlen must be
    at least every sequence's length."""
    import torch
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse, dout=dout, varlen_offsets=varlen_offsets)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bfloat16 tensor")
    if varlen_offsets is None:
        B, Nq, H, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
    else:
        T, H, d = q.shape
        Hkv = k.shape[1]
        B = varlen_offsets.numel() - 1
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with varlen offsets")
        Nq = Nk = int(max_seqlen)
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape or H % Hkv:
        raise ValueError("o and dout must be shaped like q, v like k, and Hkv must divide H")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty((fa_bwd_workspace_size(B, H, Nq) // 4,), dtype=torch.float32, device=q.device)
    st = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, Nq, Nk, d, scale, causal,
                varlen_offsets, Hkv, stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


_function = None


def _flash_attention_function():
    """The torch.autograd.Function behind flash_attention (built on first use,
    so that importing this module does not import torch)."""
    global _function
    if _function is None:
        import torch

        class FlashAttentionFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal, varlen_offsets, max_seqlen, rescale_threshold):
                o, lse = attention(q, k, v, scale, causal, varlen_offsets=varlen_offsets,
                                   max_seqlen=max_seqlen, rescale_threshold=rescale_threshold)
                extra = (varlen_offsets,) if varlen_offsets is not None else ()
                ctx.save_for_backward(q, k, v, o, lse, *extra)
                ctx.scale, ctx.causal, ctx.max_seqlen = scale, causal, max_seqlen
                return o

            @staticmethod
            def backward(ctx, dout):
                q, k, v, o, lse, *extra = ctx.saved_tensors
                dq, dk, dv = attention_bwd(q, k, v, o, lse, dout.contiguous(), ctx.scale,
                                           ctx.causal, varlen_offsets=extra[0] if extra else None,
                                           max_seqlen=ctx.max_seqlen)
                return dq, dk, dv, None, None, None, None, None

        _function = FlashAttentionFunction
    return _function


def flash_attention(q, k, v, scale: float, causal: bool, *, varlen_offsets=None, max_seqlen=None,
                    rescale_threshold: float = 8.0):
    """O = softmax(scale Q K^T) V as a differentiable torch operation: the forward
    runs fa_fwd_ex (bf16 O; LSE kept for the backward), the backward fa_bwd on
    the saved O and LSE.  Shapes as for attention(); returns o."""
    _same_gpu(q=q, k=k, v=v, varlen_offsets=varlen_offsets)
    return _flash_attention_function().apply(q, k, v, scale, causal, varlen_offsets, max_seqlen,
                                             rescale_threshold)
