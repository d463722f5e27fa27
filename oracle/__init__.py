"""fp64 CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it imports nothing from
the product path.

Two artefacts live here:

* ``oracle.c`` (loaded through ctypes): the plain three-pass softmax
  attention of the definition, computed in fp64 on whatever values the caller
  passes (the tests pass the bf16-rounded inputs widened exactly to fp64).
  See the header of ``oracle.c`` for the passages it follows.
* ``model.py``: a blockwise fp64 model of the online-softmax update with the
  conditional rescale, used only to pin the algorithm's round-by-round state;
  it is not the parity oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_default = None

_F64P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O3, OpenMP, no fast-math).

    No -march=native: the library built here may run on a different host CPU.
    """
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray, t=_F64P):
    return a.ctypes.data_as(t)


class Oracle:
    """ctypes front end over one build of oracle.c (the default one, or a test variant)."""

    def __init__(self, lib_path: str | None = None):
        if lib_path is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            lib_path = _LIB_PATH
        lib = ctypes.CDLL(lib_path)
        lib.oracle_attn_fwd.argtypes = [_F64P, _F64P, _F64P, _F64P, _F64P,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd_varlen.argtypes = [_F64P, _F64P, _F64P, _F64P, _F64P,
                                               ctypes.c_int64, _I64P, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                               ctypes.c_int]
        lib.oracle_attn_fwd_varlen.restype = ctypes.c_int
        lib.oracle_attn_fwd_rows.argtypes = [_F64P, _F64P, _F64P,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                             ctypes.c_int,
                                             _I64P, ctypes.c_int64, ctypes.c_int64, _I64P,
                                             _F64P, _F64P]
        lib.oracle_attn_fwd_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_F64P] * 7 + [ctypes.c_int64] * 6 + [ctypes.c_double,
                                                                             ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd_varlen.argtypes = [_F64P] * 7 + [ctypes.c_int64, _I64P, ctypes.c_int64,
                                                             ctypes.c_int64, ctypes.c_int64,
                                                             ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_bwd_varlen.restype = ctypes.c_int
        i64 = ctypes.c_int64
        lib.oracle_attn_bwd_rows.argtypes = [_F64P] * 4 + [i64, i64, i64, i64, ctypes.c_double,
                                                           ctypes.c_int, i64, _I64P, _F64P, i64,
                                                           _I64P, _F64P, _F64P]
        lib.oracle_attn_bwd_rows.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.oracle_num_threads())

    def attention(self, q, k, v, scale: float, causal: bool):
        """Fixed length: q [B,Nq,H,d], k/v [B,Nk,Hkv,d] (Hkv divides H)
        -> (o [B,Nq,H,d], lse [B,H,Nq])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or k.shape != v.shape or k.ndim != 4:
            raise ValueError("expected q [B,Nq,H,d] and k, v [B,Nk,Hkv,d]")
        B, Nq, H, d = q.shape
        Hkv = k.shape[2]
        if k.shape[0] != B or k.shape[3] != d or Hkv < 1 or H % Hkv:
            raise ValueError("q and k/v disagree on B or d, or Hkv does not divide H")
        Nk = k.shape[1]
        o = np.empty_like(q)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Hkv, Nq, Nk, d,
                                      float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_attn_fwd failed")
        return o, lse

    def attention_varlen(self, q, k, v, offsets, scale: float, causal: bool):
        """Packed varlen self attention: q [T,H,d], k/v [T,Hkv,d], offsets [nseq+1]
        -> (o [T,H,d], lse [H,T])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        nseq = off.shape[0] - 1
        T, H, d = q.shape
        Hkv = k.shape[1]
        if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d or Hkv < 1 or H % Hkv:
            raise ValueError("expected k, v [T,Hkv,d] with Hkv dividing H")
        if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
            raise ValueError("offsets must start at 0, be non-decreasing and end at T")
        o = np.empty_like(q)
        lse = np.empty((H, T), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse), nseq,
                                             _p(off, _I64P), H, Hkv, d, float(scale),
                                             int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_attn_fwd_varlen failed")
        return o, lse

    def attention_rows(self, q, k, v, scale: float, causal: bool, rows, offsets=None):
        """Selected rows only; rows is an int array [n, 3] of (b, h, i).

        Fixed layout when offsets is None (q [B,Nq,H,d]); otherwise packed
        varlen (q [T,H,d], b names a sequence).  Returns (o [n,d], lse [n]).
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        if offsets is None:
            _, Nq, H, d = q.shape
            Nk, Hkv = k.shape[1], k.shape[2]
            if np.any(rows[:, 0] >= q.shape[0]):
                raise ValueError("batch index out of range")
            off_p, nseq = None, 0
        else:
            off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
            _, H, d = q.shape
            Hkv = k.shape[1]
            Nq = Nk = 0
            off_p, nseq = _p(off, _I64P), off.shape[0] - 1
        o = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        if Hkv < 1 or H % Hkv:
            raise ValueError("Hkv must divide H")
        rc = self.lib.oracle_attn_fwd_rows(_p(q), _p(k), _p(v), H, Hkv, Nq, Nk, d, float(scale),
                                           int(bool(causal)), off_p, nseq, n, _p(rows, _I64P),
                                           _p(o), _p(lse))
        if rc != 0:
            raise RuntimeError("oracle_attn_fwd_rows failed (row index out of range?)")
        return o, lse


    def attention_bwd(self, q, k, v, dout, scale: float, causal: bool):
        """Gradients of O in Q, K, V for the upstream gradient dout (shaped like O).

        Fixed length: q, dout [B,Nq,H,d], k, v [B,Nk,Hkv,d] -> (dq, dk, dv)."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or dout.shape != q.shape:
            raise ValueError("expected q, dout [B,Nq,H,d] and k, v [B,Nk,Hkv,d]")
        B, Nq, H, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        if k.shape[0] != B or k.shape[3] != d or Hkv < 1 or H % Hkv:
            raise ValueError("q and k/v disagree on B or d, or Hkv does not divide H")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        rc = self.lib.oracle_attn_bwd(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv),
                                      B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_attn_bwd failed")
        return dq, dk, dv

    def attention_bwd_varlen(self, q, k, v, dout, offsets, scale: float, causal: bool):
        """Packed varlen gradients: q, dout [T,H,d], k, v [T,Hkv,d] -> (dq, dk, dv)."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        T, H, d = q.shape
        Hkv = k.shape[1]
        if k.shape != v.shape or k.shape[0] != T or dout.shape != q.shape or Hkv < 1 or H % Hkv:
            raise ValueError("expected q, dout [T,H,d] and k, v [T,Hkv,d]")
        if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
            raise ValueError("offsets must start at 0, be non-decreasing and end at T")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        rc = self.lib.oracle_attn_bwd_varlen(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk),
                                             _p(dv), off.shape[0] - 1, _p(off, _I64P), H, Hkv, d,
                                             float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError("oracle_attn_bwd_varlen failed")
        return dq, dk, dv

    def attention_bwd_rows(self, q, k, v, dout, scale: float, causal: bool, qrows, krows):
        """Selected gradient rows of one (batch, K/V head) with its G query heads.

        q, dout [Nq,G,d]; k, v [Nk,d]; qrows: (g, i) pairs; krows: key indices.
        Returns (dq [len(qrows),d], dk [len(krows),d], dv [len(krows),d])."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        if q.ndim != 3 or k.ndim != 2 or k.shape != v.shape or dout.shape != q.shape or \
                k.shape[1] != q.shape[2]:
            raise ValueError("expected q, dout [Nq,G,d] and k, v [Nk,d]")
        Nq, G, d = q.shape
        Nk = k.shape[0]
        qr = np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1, 2))
        kr = np.ascontiguousarray(np.asarray(krows, dtype=np.int64).reshape(-1))
        dq = np.zeros((qr.shape[0], d))
        dk = np.zeros((kr.shape[0], d))
        dv = np.zeros((kr.shape[0], d))
        rc = self.lib.oracle_attn_bwd_rows(_p(q), _p(k), _p(v), _p(dout), G, Nq, Nk, d,
                                           float(scale), int(bool(causal)), qr.shape[0],
                                           _p(qr, _I64P), _p(dq), kr.shape[0], _p(kr, _I64P),
                                           _p(dk), _p(dv))
        if rc != 0:
            raise RuntimeError("oracle_attn_bwd_rows failed (bad row index or allocation)")
        return dq, dk, dv


def default() -> Oracle:
    """The oracle built from oracle.c in this directory (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(q, k, v, scale: float, causal: bool):
    return default().attention(q, k, v, scale, causal)


def attention_varlen(q, k, v, offsets, scale: float, causal: bool):
    return default().attention_varlen(q, k, v, offsets, scale, causal)


def attention_rows(q, k, v, scale: float, causal: bool, rows, offsets=None):
    return default().attention_rows(q, k, v, scale, causal, rows, offsets)


def attention_bwd(q, k, v, dout, scale: float, causal: bool):
    return default().attention_bwd(q, k, v, dout, scale, causal)


def attention_bwd_varlen(q, k, v, dout, offsets, scale: float, causal: bool):
    return default().attention_bwd_varlen(q, k, v, dout, offsets, scale, causal)


def attention_bwd_rows(q, k, v, dout, scale: float, causal: bool, qrows, krows):
    return default().attention_bwd_rows(q, k, v, dout, scale, causal, qrows, krows)
