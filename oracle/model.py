"""Blockwise fp64 model of the online-softmax forward update -- TEST INFRASTRUCTURE ONLY.

This is not the parity oracle (that is the three-pass definition in
``oracle.c``).  It walks the K/V blocks of one head in the order and notation
of the pages, so the tests can pin the algorithm's state round by round:

* "Flash Attention 4" (mlc.ai), section "algorithm structure": per-row state
  row_max (reference r_i, not necessarily the true maximum), row_sum (l_i) and
  the unnormalised accumulator O; scale_log2 = log2(e) * scale; candidate =
  max(row_max, rowmax(S)); on the first block the candidate is taken with
  acc_scale = 1; later, delta = (row_max - candidate) * scale_log2 and the old
  reference is kept while delta >= -threshold (acc_scale = 1), else the
  candidate is taken and acc_scale = exp2(delta); row_max_safe is 0 when the
  reference is -inf; P = exp2((S - row_max_safe) * scale_log2); row_sum =
  row_sum * acc_scale + rowsum(P); O = O * acc_scale + P V; at the end
  O / row_sum (0 when row_sum is 0).
* same page, section "rescale and write-back": LSE = ln(row_sum) + r * scale for
  any consistent reference r, -inf for a row with no valid key.
* "FlashAttention：一次前向计算" (qingsen), section "general update": the
  always-rescale form (threshold 0) with m, alpha, l and O per round.
* same page, section "causal mask": masked scores are set to -inf before the
  maximum and the exponent.

Reading where the pages leave a case open: on a later block whose candidate
is still -inf (every key so far masked), delta would be (-inf) - (-inf); the
model keeps the reference (-inf) with acc_scale = 1, so the all-zero state
stays zero, which is what the page's row_max_safe guard is for.
"""
from __future__ import annotations

import math

import numpy as np


def fa4_forward(q, k, v, scale: float, causal: bool = False, block_n: int = 128,
                threshold: float = 8.0, reverse: bool = False, trace: bool = False,
                tie_eps: float = 1e-3):
    """One head: q [Nq, d], k/v [Nk, d] -> dict(o, lse, rescales, rescale_rows,
    near_ties, trace).

    ``threshold`` is tau (8 = conditional rescale, 0 = always rescale);
    ``reverse`` walks the K/V blocks from last to first.  ``rescales`` counts
    (row, block) pairs where the reference was switched after the first block;
    ``rescale_rows`` is that count per row, and ``near_ties`` per row the number
    of such later blocks whose decision was within ``tie_eps`` of the threshold:
    the decision compares the block's maximum with the reference, so the margin
    is |(row_max - block max) * scale_log2 + threshold| (both finite); there an
    fp32 evaluation of the same scores may decide the other way.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, d = q.shape
    Nk = k.shape[0]
    scale_log2 = float(scale) * math.log2(math.e)

    row_max = np.full(Nq, -np.inf)
    row_sum = np.zeros(Nq)
    O = np.zeros((Nq, v.shape[1]))
    first = True
    rescales = 0
    rescale_rows = np.zeros(Nq, dtype=np.int64)
    near_ties = np.zeros(Nq, dtype=np.int64)
    states = []

    nblocks = (Nk + block_n - 1) // block_n
    order = range(nblocks - 1, -1, -1) if reverse else range(nblocks)
    qi = np.arange(Nq)[:, None]
    for blk in order:
        j0, j1 = blk * block_n, min(Nk, (blk + 1) * block_n)
        S = q @ k[j0:j1].T                      # unscaled scores
        if causal:
            kj = np.arange(j0, j1)[None, :]
            S = np.where(kj > qi + (Nk - Nq), -np.inf, S)
        candidate = np.maximum(row_max, S.max(axis=1))
        if first:
            new_ref = candidate
            acc_scale = np.ones(Nq)
        else:
            with np.errstate(invalid="ignore"):
                delta = (row_max - candidate) * scale_log2
            keep = (candidate == -np.inf) | (delta >= -threshold)
            new_ref = np.where(keep, row_max, candidate)
            with np.errstate(invalid="ignore"):
                acc_scale = np.where(keep, 1.0, np.exp2(np.where(keep, 0.0, delta)))
            rescales += int(np.count_nonzero(~keep))
            rescale_rows += ~keep
            bmax = S.max(axis=1)
            both = np.isfinite(row_max) & np.isfinite(bmax)
            with np.errstate(invalid="ignore"):
                gap = np.where(both, (row_max - bmax) * scale_log2, np.inf)
            near_ties += both & (np.abs(gap + threshold) < tie_eps)
        row_max_safe = np.where(new_ref == -np.inf, 0.0, new_ref)
        P = np.exp2((S - row_max_safe[:, None]) * scale_log2)
        row_sum = row_sum * acc_scale + P.sum(axis=1)
        block_O = P @ v[j0:j1]
        O = block_O if first else O * acc_scale[:, None] + block_O
        row_max = new_ref
        first = False
        if trace:
            states.append(dict(block=blk, row_max=row_max.copy(), acc_scale=acc_scale.copy(),
                               P=P.copy(), row_sum=row_sum.copy(), O=O.copy()))

    nz = row_sum != 0
    out = np.zeros_like(O)
    out[nz] = O[nz] / row_sum[nz, None]
    lse = np.full(Nq, -np.inf)
    lse[nz] = np.log(row_sum[nz]) + row_max[nz] * float(scale)
    return dict(o=out, lse=lse, rescales=rescales, rescale_rows=rescale_rows,
                near_ties=near_ties, trace=states)


def update_row(row_max: float, row_sum: float, O, S, V, scale_log2: float,
               threshold: float = 8.0, first_block: bool = False):
    """One block of the update for a single row with explicit prior state.

    Returns (candidate, delta, new_ref, acc_scale, P, row_sum, O) in the
    variable names of the "algorithm structure" pseudocode of the FA4 page.
    """
    S = np.asarray(S, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    candidate = max(row_max, float(S.max()))
    if first_block:
        delta, new_ref, acc_scale = 0.0, candidate, 1.0
    else:
        delta = (row_max - candidate) * scale_log2 if candidate != -math.inf else 0.0
        if candidate == -math.inf or delta >= -threshold:
            new_ref, acc_scale = row_max, 1.0
        else:
            new_ref, acc_scale = candidate, 2.0 ** delta
    safe = 0.0 if new_ref == -math.inf else new_ref
    P = np.exp2((S - safe) * scale_log2)
    new_sum = row_sum * acc_scale + float(P.sum())
    new_O = O * acc_scale + P @ V
    return candidate, delta, new_ref, acc_scale, P, new_sum, new_O
