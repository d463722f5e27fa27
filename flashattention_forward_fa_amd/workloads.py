"""Seeded synthetic inputs for the attention forward pass.

This module only draws and packages inputs: it holds none of the attention
arithmetic, imports neither the HIP binding nor the CPU reference, and is the
one piece of code that the tests, the benchmark and the reference checks share.

Recipe (every draw is seeded, ``numpy.random.default_rng`` / PCG64):

* Q, K, V are drawn as float32 ``standard_normal`` in full C order, in the order
  Q, K, V, and rounded to bf16 with round-to-nearest-even.
* Fixed-length tensors use the [batch, sequence, head, dim] layout.
* Outlier keys: after V, for each (batch, head) independently, ``round(frac*Nk)``
  distinct key positions are drawn without replacement and those K rows are
  multiplied by ``outlier_scale`` (8 is a power of two, so bf16 stays exact).
  This forces jumps of the row maximum, i.e. rescale events.
* Variable length: the sequence lengths are drawn first, as integers uniform on
  an inclusive range, then Q, K, V of shape [T, head, dim] with T = sum(L); the
  int32 cumulative offsets [0, L0, L0+L1, ...] describe the packing.
* Grouped K/V heads: K and V are drawn with Hkv heads ([.., Hkv, dim]); with
  Hkv = H the draws are the multi-head ones.
* The backward's upstream gradient dO: standard_normal shaped like O, from its
  own seed, rounded to bf16.

The named workloads mirror the five synthetic configurations the method is
measured on (seed = 1000 + number).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


# ---------------------------------------------------------------- bf16 bits

def bf16_bits(x) -> np.ndarray:
    """float32 values -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    return bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- workloads

@dataclass
class Workload:
    """One synthetic problem: bf16 bit patterns plus its shape description."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    scale: float
    o_dtype: str                     # "bf16" or "f32"
    seed: int
    q: np.ndarray                    # uint16 bits
    k: np.ndarray
    v: np.ndarray
    offsets: Optional[np.ndarray] = None   # int32 [B+1] for packed varlen
    lengths: Optional[np.ndarray] = None
    notes: dict = field(default_factory=dict)
    Hkv: Optional[int] = None        # K/V heads; None = H

    @property
    def varlen(self) -> bool:
        return self.offsets is not None

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1]) if self.varlen else self.B * self.Nq

    def flops(self) -> float:
        """Attention forward flops: 4*B*H*Nq*Nk*d, halved when causal."""
        if self.varlen:
            per = sum(4.0 * self.H * float(L) * float(L) * self.d for L in self.lengths)
        else:
            per = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return per / 2.0 if self.causal else per

    def io_bytes(self) -> int:
        """Algorithmic minimum HBM bytes: read Q, K, V once, write O and LSE once."""
        osz = 4 if self.o_dtype == "f32" else 2
        if self.varlen:
            T = self.total_tokens
            return T * self.H * self.d * (2 + osz) + 2 * T * self.kv_heads * self.d * 2 \
                + T * self.H * 4
        qo = self.B * self.Nq * self.H
        kv = self.B * self.Nk * self.kv_heads
        return qo * self.d * (2 + osz) + 2 * kv * self.d * 2 + qo * 4

    def describe(self) -> dict:
        dsc = dict(workload=self.name, batch=self.B, heads=self.H, seq_q=self.Nq, seq_k=self.Nk,
                   head_dim=self.d, causal=self.causal, scale=self.scale, o_dtype=self.o_dtype,
                   seed=self.seed)
        if self.Hkv is not None and self.Hkv != self.H:
            dsc.update(kv_heads=self.Hkv)
        if self.varlen:
            dsc.update(lengths=[int(x) for x in self.lengths], total_tokens=self.total_tokens)
        dsc.update(self.notes)
        return dsc


def _draw_qkv(rng, shape_q, shape_kv):
    q = rng.standard_normal(shape_q, dtype=np.float32)
    k = rng.standard_normal(shape_kv, dtype=np.float32)
    v = rng.standard_normal(shape_kv, dtype=np.float32)
    return q, k, v


def make_fixed(B, H, Nq, Nk, d, *, seed, causal, scale=None, o_dtype="bf16",
               outlier_frac=0.0, outlier_scale=8.0, name=None, Hkv=None) -> Workload:
    """Fixed-length inputs, q [B, Nq, H, d] and k, v [B, Nk, Hkv, d] (Hkv = H
    unless given), drawn i.i.d. N(0,1) and rounded to bf16."""
    rng = np.random.default_rng(seed)
    hk = H if Hkv is None else Hkv
    q, k, v = _draw_qkv(rng, (B, Nq, H, d), (B, Nk, hk, d))
    notes = {}
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * Nk))
        for b in range(B):
            for h in range(hk):
                pos = rng.choice(Nk, n_out, replace=False)
                k[b, pos, h, :] *= np.float32(outlier_scale)
        notes = dict(outlier_rows_per_head=n_out, outlier_scale=outlier_scale)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kvs = "" if Hkv is None or Hkv == H else f"_Hkv{Hkv}"
    return Workload(name or f"B{B}_H{H}{kvs}_Nq{Nq}_Nk{Nk}_d{d}_{'causal' if causal else 'full'}",
                    B, H, Nq, Nk, d, bool(causal), float(scale), o_dtype, seed,
                    bf16_bits(q), bf16_bits(k), bf16_bits(v), notes=notes, Hkv=Hkv)


def make_varlen(H, d, *, seed, causal=True, lengths=None, nseq=16, len_lo=128, len_hi=8192,
                scale=None, o_dtype="bf16", name=None, Hkv=None) -> Workload:
    """Packed inputs, q [T, H, d] and k, v [T, Hkv, d]; lengths drawn uniform on
    [len_lo, len_hi] unless given."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(len_lo, len_hi, nseq, endpoint=True)
    lengths = np.asarray(lengths, dtype=np.int64)
    offsets = np.zeros(len(lengths) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    T = int(offsets[-1])
    hk = H if Hkv is None else Hkv
    q, k, v = _draw_qkv(rng, (T, H, d), (T, hk, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    maxlen = int(lengths.max()) if len(lengths) else 0
    return Workload(name or f"varlen{len(lengths)}_H{H}_d{d}", len(lengths), H, maxlen, maxlen,
                    d, bool(causal), float(scale), o_dtype, seed,
                    bf16_bits(q), bf16_bits(k), bf16_bits(v),
                    offsets=offsets.astype(np.int32), lengths=lengths, Hkv=Hkv)


def make_dout(w: Workload, seed: int) -> np.ndarray:
    """Upstream gradient dO for workload w (the backward's input): bf16 bits of
    float32 standard_normal draws shaped like O ([B,Nq,H,d] or [T,H,d])."""
    rng = np.random.default_rng(seed)
    shape = (w.total_tokens, w.H, w.d) if w.varlen else (w.B, w.Nq, w.H, w.d)
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


CONFIG_NAMES = {
    1: "noncausal_B1_H2_N256_d64_f32out",
    2: "noncausal_B4_H16_N2048_d128",
    3: "causal_B2_H32_N4096_d128",
    4: "causal_B1_H16_N16384_d128_outlierK",
    5: "varlen_causal_16seq_L128-8192_H32_d64",
}


def config(n: int) -> Workload:
    """The five measured configurations (seed 1000 + n)."""
    seed = 1000 + n
    if n == 1:
        return make_fixed(1, 2, 256, 256, 64, seed=seed, causal=False, scale=1.0 / 8.0,
                          o_dtype="f32", name=CONFIG_NAMES[1])
    if n == 2:
        return make_fixed(4, 16, 2048, 2048, 128, seed=seed, causal=False,
                          scale=1.0 / math.sqrt(128), name=CONFIG_NAMES[2])
    if n == 3:
        return make_fixed(2, 32, 4096, 4096, 128, seed=seed, causal=True,
                          scale=1.0 / math.sqrt(128), name=CONFIG_NAMES[3])
    if n == 4:
        return make_fixed(1, 16, 16384, 16384, 128, seed=seed, causal=True,
                          scale=1.0 / math.sqrt(128), outlier_frac=0.01, outlier_scale=8.0,
                          name=CONFIG_NAMES[4])
    if n == 5:
        return make_varlen(32, 64, seed=seed, causal=True, nseq=16, len_lo=128, len_hi=8192,
                           scale=1.0 / 8.0, name=CONFIG_NAMES[5])
    raise ValueError(f"no configuration {n}")


def grouped(n: int, kv_heads: int) -> Workload:
    """A fixed-length configuration (2, 3 or 4) with K/V drawn for kv_heads heads
    (grouped-query attention; same query shape, flops and seed)."""
    base = {2: (4, 16, 2048, False, 0.0), 3: (2, 32, 4096, True, 0.0),
            4: (1, 16, 16384, True, 0.01)}
    if n not in base:
        raise ValueError(f"no grouped variant of configuration {n}")
    B, H, N, causal, frac = base[n]
    return make_fixed(B, H, N, N, 128, seed=1000 + n, causal=causal, scale=1.0 / math.sqrt(128),
                      outlier_frac=frac, outlier_scale=8.0, Hkv=kv_heads,
                      name=f"{CONFIG_NAMES[n]}_Hkv{kv_heads}")
