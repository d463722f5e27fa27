"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the pages' printed values, closed forms derived from the
definition, an independent library implementation (torch's fp64 CPU
scaled-dot-product attention, scipy's logsumexp), or an invariant of softmax
attention.  ``tests/test_oracle.py`` runs them on the real oracle and
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies to show
that each planted mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _frac(x):
    return np.asarray(x, dtype=np.float64)[..., 0] / np.asarray(x, dtype=np.float64)[..., 1]


def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example_two_rounds.json")) as f:
        g = json.load(f)
    g["Q"] = np.array(g["Q"], dtype=np.float64)
    g["K"] = np.array(g["K"], dtype=np.float64)
    g["V"] = np.array(g["V"], dtype=np.float64)
    return g


def _one_head(x):
    """[N, d] -> [1, N, 1, d]"""
    return np.asarray(x, dtype=np.float64)[None, :, None, :]


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    ok = same_inf | (np.abs(a - b) <= tol * np.maximum(1.0, np.abs(b)))
    assert np.all(ok), f"{what}: max diff {np.nanmax(np.abs(np.where(same_inf, 0, a - b)))}"


# ------------------------------------------------------------ printed values

def pin_worked_example(orc):
    """Non-causal 2x4 example with s = ln 2: final O (figure 10) and LSE = (ln 8, ln 9)."""
    g = load_worked_example()
    o, lse = orc.attention(_one_head(g["Q"]), _one_head(g["K"]), _one_head(g["V"]),
                           math.log(2.0), False)
    _close(o[0, :, 0, :], _frac(g["final"]["O"]), what="O")
    _close(lse[0, 0], [math.log(8.0), math.log(9.0)], what="LSE")


def pin_causal_figure12(orc):
    """Causal scores of figure 12 (row 0 keeps key 0, row 1 keeps keys 0-1), Nq = Nk = 2.

    Closed forms from the definition: O_0 = V_0 = (1, 0), LSE_0 = s*0 = 0;
    weights of row 1 are 2^1, 2^0 -> O_1 = (2/3, 1/3), LSE_1 = ln 3.
    """
    g = load_worked_example()
    o, lse = orc.attention(_one_head(g["Q"]), _one_head(g["K"][:2]), _one_head(g["V"][:2]),
                           math.log(2.0), True)
    _close(o[0, :, 0, :], [[1.0, 0.0], [2.0 / 3.0, 1.0 / 3.0]], what="O")
    _close(lse[0, 0], [0.0, math.log(3.0)], what="LSE")


def pin_bottom_right_alignment(orc):
    """Nq = 2 queries against Nk = 4 keys, causal, bottom-right aligned (FA4 page).

    Query 0 may use keys 0..2: weights 1, 2, 4 -> O_0 = (5/7, 6/7), LSE_0 = ln 7.
    Query 1 may use keys 0..3, the non-causal row of figure 10: (4/3, 1/3), ln 9.
    """
    g = load_worked_example()
    o, lse = orc.attention(_one_head(g["Q"]), _one_head(g["K"]), _one_head(g["V"]),
                           math.log(2.0), True)
    _close(o[0, :, 0, :], [[5.0 / 7.0, 6.0 / 7.0], [4.0 / 3.0, 1.0 / 3.0]], what="O")
    _close(lse[0, 0], [math.log(7.0), math.log(9.0)], what="LSE")


def pin_exercise7_bounds(orc):
    """FA4 page, exercise 7: Nq = 6, Nk = 8, bottom-right causal mask.

    With q = 0 every valid key gets the same weight and V = I makes O row i the
    indicator of its valid keys divided by their count: query i sees keys
    0..i+2, so query 0 ends at key 2 and query 5 at key 7.
    """
    Nq, Nk = 6, 8
    q = np.zeros((Nq, Nk))
    k = np.arange(Nk * Nk, dtype=np.float64).reshape(Nk, Nk) * 0.25
    v = np.eye(Nk)
    o, lse = orc.attention(_one_head(q), _one_head(k), _one_head(v), 0.7, True)
    for i in range(Nq):
        n = i + 3
        want = np.zeros(Nk)
        want[:n] = 1.0 / n
        _close(o[0, i, 0], want, what=f"row {i}")
        _close(lse[0, 0, i], math.log(n), what=f"lse {i}")


# ------------------------------------------------------------ library routine

def _torch_reference(q, k, v, scale, causal):
    """torch's fp64 CPU SDPA (its own grouped-head handling when k/v have fewer
    heads) and scipy's logsumexp over explicitly repeated key heads."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp
    Nq, Nk = q.shape[1], k.shape[1]
    H, Hkv = q.shape[2], k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()   # [B,H,N,d]
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous()
    mask = None
    allowed = np.ones((Nq, Nk), dtype=bool)
    if causal:
        allowed = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        mask = torch.from_numpy(allowed)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                       enable_gqa=(H != Hkv))
    o = o.permute(0, 2, 1, 3).numpy()
    kr = np.repeat(k, H // Hkv, axis=2)
    s = scale * np.einsum("bqhd,bkhd->bhqk", q, kr)
    s = np.where(allowed[None, None], s, -np.inf)
    lse = logsumexp(s, axis=-1)
    return o, lse


def pin_torch_sdpa(orc):
    """Random tiny problems vs torch's fp64 CPU scaled_dot_product_attention and scipy logsumexp."""
    rng = np.random.default_rng(7)
    shapes = [(2, 3, 5, 7, 4, False), (2, 3, 5, 7, 4, True), (1, 2, 9, 9, 8, True),
              (3, 1, 4, 11, 6, True), (1, 4, 13, 6, 5, False), (2, 2, 16, 16, 16, True)]
    for (B, H, Nq, Nk, d, causal) in shapes:
        q = rng.standard_normal((B, Nq, H, d))
        k = rng.standard_normal((B, Nk, H, d))
        v = rng.standard_normal((B, Nk, H, d))
        scale = 0.37 + 0.1 * d
        o, lse = orc.attention(q, k, v, scale, causal)
        ro, rlse = _torch_reference(q, k, v, scale, causal)
        _close(o, ro, tol=1e-12, what=f"O {B, H, Nq, Nk, d, causal}")
        _close(lse, rlse, tol=1e-12, what=f"LSE {B, H, Nq, Nk, d, causal}")


def pin_torch_sdpa_grouped_heads(orc):
    """Grouped K/V heads (Hkv < H, MQA at Hkv = 1) vs torch's SDPA with enable_gqa."""
    rng = np.random.default_rng(8)
    shapes = [(2, 4, 2, 5, 7, 4, False), (1, 6, 3, 9, 9, 8, True), (2, 4, 1, 6, 11, 5, True),
              (1, 8, 2, 13, 6, 3, False)]
    for (B, H, Hkv, Nq, Nk, d, causal) in shapes:
        q = rng.standard_normal((B, Nq, H, d))
        k = rng.standard_normal((B, Nk, Hkv, d))
        v = rng.standard_normal((B, Nk, Hkv, d))
        o, lse = orc.attention(q, k, v, 0.41, causal)
        ro, rlse = _torch_reference(q, k, v, 0.41, causal)
        _close(o, ro, tol=1e-12, what=f"O {B, H, Hkv, Nq, Nk, d, causal}")
        _close(lse, rlse, tol=1e-12, what=f"LSE {B, H, Hkv, Nq, Nk, d, causal}")


def load_gqa_exercise():
    with open(os.path.join(GOLDEN, "gqa_exercise8.json")) as f:
        return json.load(f)


def pin_gqa_exercise8(orc):
    """The page's head grouping (exercise 8: 32 query heads, 8 K/V heads): query
    heads kv*G .. kv*G+G-1 read K/V head kv.  Each K/V head c carries V = c + 1
    and K = 0 (uniform weights), so O of query head h is 1 + (the K/V head it read)."""
    g = load_gqa_exercise()
    H, Hkv = g["num_qo_heads"], g["num_kv_heads"]
    G = g["GQA_RATIO"]
    assert H // Hkv == G and g["BLK_M"] // G == g["SEQ_Q_PER_TILE"]
    N, d = 3, 2
    q = np.ones((1, N, H, d))
    k = np.zeros((1, N, Hkv, d))
    v = np.broadcast_to((np.arange(Hkv, dtype=np.float64) + 1.0)[None, None, :, None],
                        (1, N, Hkv, d)).copy()
    for causal in (False, True):
        o, _ = orc.attention(q, k, v, 0.5, causal)
        kv_read = o[0, :, :, 0] - 1.0                 # [N, H]
        for row, (seq, head) in g["packed_rows"].items():
            row = int(row)
            assert row // G == seq and g["kv_head_idx"] * G + row % G == head
            _close(kv_read[:, head], np.full(N, g["kv_head_idx"]), what=f"head {head}")
        _close(kv_read, np.broadcast_to(np.arange(H) // G, (N, H)), what="all heads")
        # varlen layout, same grouping
        ov, _ = orc.attention_varlen(q[0], k[0], v[0], [0, N], 0.5, causal)
        _close(ov[:, :, 0] - 1.0, np.broadcast_to(np.arange(H) // G, (N, H)), what="varlen heads")


def pin_gqa_equals_repeated_heads(orc):
    """Grouped K/V heads give exactly the multi-head result on K/V with each head
    repeated G times consecutively (fixed, varlen and selected rows)."""
    rng = np.random.default_rng(9)
    B, H, Hkv, Nq, Nk, d = 2, 6, 2, 5, 8, 4
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    kr, vr = np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2)
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, 0.55, causal)
        o1, l1 = orc.attention(q, kr, vr, 0.55, causal)
        _close(o, o1, what="O")
        _close(lse, l1, what="LSE")
        rows = np.array([[0, 5, 4], [1, 2, 0], [1, 3, 2]])
        ro, rl = orc.attention_rows(q, k, v, 0.55, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            _close(ro[n], o[b, i, h], what=f"row {n}")
            _close(rl[n], lse[b, h, i], what=f"lse {n}")
    lengths = [3, 6]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = off[-1]
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    o, lse = orc.attention_varlen(q, k, v, off, 0.55, True)
    o1, l1 = orc.attention_varlen(q, kr, vr, off, 0.55, True)
    _close(o, o1, what="varlen O")
    _close(lse, l1, what="varlen LSE")
    rows = np.array([[1, 4, 5], [0, 1, 2]])
    ro, rl = orc.attention_rows(q, k, v, 0.55, True, rows, offsets=off)
    for n, (b, h, i) in enumerate(rows):
        _close(ro[n], o[off[b] + i, h], what=f"varlen row {n}")
        _close(rl[n], lse[h, off[b] + i], what=f"varlen lse {n}")


# ------------------------------------------------------------ invariants

def pin_rows_sum_to_one(orc):
    """With V = I (Nk = d) O equals the weight matrix P: non-negative rows summing to 1."""
    rng = np.random.default_rng(11)
    Nq, Nk = 7, 10
    q = rng.standard_normal((Nq, Nk))
    k = rng.standard_normal((Nk, Nk))
    for causal in (False, True):
        o, _ = orc.attention(_one_head(q), _one_head(k), _one_head(np.eye(Nk)), 0.8, causal)
        p = o[0, :, 0, :]
        assert np.all(p >= 0.0)
        _close(p.sum(axis=1), np.ones(Nq), what="row sums")


def pin_shift_invariance(orc):
    """Adding the same constant to every score of a row leaves O alone and shifts LSE.

    An extra dimension with q = 1 and k = c adds s*c to each score of every row.
    """
    rng = np.random.default_rng(12)
    Nq, Nk, d = 6, 9, 4
    q = rng.standard_normal((Nq, d))
    k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    s, c = 0.6, 5.0
    o0, l0 = orc.attention(_one_head(q), _one_head(k), _one_head(v), s, False)
    q1 = np.concatenate([q, np.ones((Nq, 1))], axis=1)
    k1 = np.concatenate([k, np.full((Nk, 1), c)], axis=1)
    v1 = np.concatenate([v, np.zeros((Nk, 1))], axis=1)
    o1, l1 = orc.attention(_one_head(q1), _one_head(k1), _one_head(v1), s, False)
    _close(o1[..., :d], o0, tol=1e-12, what="O")
    _close(l1, l0 + s * c, tol=1e-12, what="LSE")


def pin_causal_row0(orc):
    """Causal self attention: row 0 sees only key 0, so O_0 = V_0 and LSE_0 = s*q0.k0."""
    rng = np.random.default_rng(13)
    B, H, N, d = 2, 3, 8, 4
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    o, lse = orc.attention(q, k, v, 0.5, True)
    _close(o[:, 0], v[:, 0], what="O_0")
    _close(lse[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), what="LSE_0")


def pin_convex_hull(orc):
    """Each output coordinate lies between the min and max of the valid value rows."""
    rng = np.random.default_rng(14)
    N, d = 12, 6
    q = rng.standard_normal((N, d)) * 3
    k = rng.standard_normal((N, d)) * 3
    v = rng.standard_normal((N, d))
    o, _ = orc.attention(_one_head(q), _one_head(k), _one_head(v), 1.0, True)
    for i in range(N):
        lo = v[: i + 1].min(axis=0) - 1e-12
        hi = v[: i + 1].max(axis=0) + 1e-12
        assert np.all(o[0, i, 0] >= lo) and np.all(o[0, i, 0] <= hi), f"row {i}"


def pin_future_independence(orc):
    """Causal row i does not depend on key/value rows after i."""
    rng = np.random.default_rng(15)
    N, d = 10, 4
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o0, l0 = orc.attention(_one_head(q), _one_head(k), _one_head(v), 0.9, True)
    cut = 4
    k2, v2 = k.copy(), v.copy()
    k2[cut + 1:] = rng.standard_normal((N - cut - 1, d)) * 10
    v2[cut + 1:] = rng.standard_normal((N - cut - 1, d)) * 10
    o1, l1 = orc.attention(_one_head(q), _one_head(k2), _one_head(v2), 0.9, True)
    _close(o1[0, : cut + 1], o0[0, : cut + 1], what="O")
    _close(l1[0, 0, : cut + 1], l0[0, 0, : cut + 1], what="LSE")
    assert np.max(np.abs(o1[0, cut + 1:] - o0[0, cut + 1:])) > 1e-3


def pin_scale_zero_mean(orc):
    """scale = 0: every valid key gets weight 1/n, O is the mean of the valid V rows, LSE = ln n."""
    rng = np.random.default_rng(16)
    Nq, Nk, d = 5, 8, 3
    q = rng.standard_normal((Nq, d))
    k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    o, lse = orc.attention(_one_head(q), _one_head(k), _one_head(v), 0.0, True)
    for i in range(Nq):
        n = i + Nk - Nq + 1
        _close(o[0, i, 0], v[:n].mean(axis=0), what=f"row {i}")
        _close(lse[0, 0, i], math.log(n), what=f"lse {i}")


def pin_rows_without_keys(orc):
    """Causal with Nq > Nk: the first Nq - Nk rows have no valid key -> O = 0, LSE = -inf."""
    rng = np.random.default_rng(17)
    Nq, Nk, d = 7, 3, 4
    q = rng.standard_normal((Nq, d))
    k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    o, lse = orc.attention(_one_head(q), _one_head(k), _one_head(v), 0.5, True)
    assert np.all(o[0, : Nq - Nk] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, : Nq - Nk]))
    _close(o[0, Nq - Nk, 0], v[0], what="first row with a key")
    assert np.all(np.isfinite(lse[0, 0, Nq - Nk:]))


def pin_key_permutation(orc):
    """Non-causal: permuting key and value rows together changes nothing."""
    rng = np.random.default_rng(18)
    Nq, Nk, d = 6, 11, 5
    q = rng.standard_normal((2, Nq, 3, d))
    k = rng.standard_normal((2, Nk, 3, d))
    v = rng.standard_normal((2, Nk, 3, d))
    perm = rng.permutation(Nk)
    o0, l0 = orc.attention(q, k, v, 0.7, False)
    o1, l1 = orc.attention(q, k[:, perm], v[:, perm], 0.7, False)
    _close(o1, o0, what="O")
    _close(l1, l0, what="LSE")


def pin_head_batch_slices(orc):
    """Each (batch, head) of a batched call equals a single-head call on that slice."""
    rng = np.random.default_rng(19)
    B, H, Nq, Nk, d = 2, 3, 5, 6, 4
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    v = rng.standard_normal((B, Nk, H, d))
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, 0.45, causal)
        for b in range(B):
            for h in range(H):
                o1, l1 = orc.attention(_one_head(q[b, :, h]), _one_head(k[b, :, h]),
                                       _one_head(v[b, :, h]), 0.45, causal)
                _close(o[b, :, h], o1[0, :, 0], what=f"O {b},{h}")
                _close(lse[b, h], l1[0, 0], what=f"LSE {b},{h}")


def pin_varlen_is_per_sequence(orc):
    """A packed varlen call equals separate calls on each sequence."""
    rng = np.random.default_rng(20)
    lengths = [3, 1, 7, 5]
    H, d = 2, 4
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = off[-1]
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    for causal in (False, True):
        o, lse = orc.attention_varlen(q, k, v, off, 0.6, causal)
        for b, L in enumerate(lengths):
            sl = slice(off[b], off[b + 1])
            o1, l1 = orc.attention(q[None, sl], k[None, sl], v[None, sl], 0.6, causal)
            _close(o[sl], o1[0], what=f"O seq {b}")
            _close(lse[:, sl], l1[0], what=f"LSE seq {b}")


def pin_rows_match_full(orc):
    """The selected-rows entry point returns the same rows as the full call (fixed and varlen)."""
    rng = np.random.default_rng(21)
    B, H, Nq, Nk, d = 2, 3, 6, 9, 4
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    v = rng.standard_normal((B, Nk, H, d))
    o, lse = orc.attention(q, k, v, 0.3, True)
    rows = np.array([[0, 0, 0], [1, 2, 5], [0, 1, 3], [1, 0, 4]])
    ro, rl = orc.attention_rows(q, k, v, 0.3, True, rows)
    for n, (b, h, i) in enumerate(rows):
        _close(ro[n], o[b, i, h], what=f"row {n}")
        _close(rl[n], lse[b, h, i], what=f"lse {n}")
    lengths = [4, 2, 6]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = off[-1]
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    o, lse = orc.attention_varlen(q, k, v, off, 0.3, True)
    rows = np.array([[0, 0, 3], [1, 2, 1], [2, 1, 5], [2, 0, 0]])
    ro, rl = orc.attention_rows(q, k, v, 0.3, True, rows, offsets=off)
    for n, (b, h, i) in enumerate(rows):
        _close(ro[n], o[off[b] + i, h], what=f"varlen row {n}")
        _close(rl[n], lse[h, off[b] + i], what=f"varlen lse {n}")


# ------------------------------------------------------------ backward

def _torch_grads(q, k, v, dout, scale, causal):
    """Gradients from torch's fp64 CPU autograd through its SDPA (a library routine)."""
    import torch
    import torch.nn.functional as F
    Nq, Nk = q.shape[1], k.shape[1]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous().requires_grad_()
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous().requires_grad_()
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous().requires_grad_()
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                       enable_gqa=(q.shape[2] != k.shape[2]))
    o.backward(torch.from_numpy(dout).permute(0, 2, 1, 3).contiguous())
    return tuple(t.grad.permute(0, 2, 1, 3).numpy() for t in (tq, tk, tv))


def pin_bwd_torch_autograd(orc):
    """dQ, dK, dV vs torch's fp64 autograd of SDPA (grouped heads, Nq != Nk, causal)."""
    rng = np.random.default_rng(30)
    shapes = [(2, 3, 3, 5, 7, 4, False), (1, 4, 2, 9, 9, 8, True), (2, 4, 1, 6, 11, 5, True),
              (1, 2, 2, 12, 6, 3, False)]
    for (B, H, Hkv, Nq, Nk, d, causal) in shapes:
        if causal and Nq > Nk:
            continue
        q = rng.standard_normal((B, Nq, H, d))
        k = rng.standard_normal((B, Nk, Hkv, d))
        v = rng.standard_normal((B, Nk, Hkv, d))
        do = rng.standard_normal((B, Nq, H, d))
        got = orc.attention_bwd(q, k, v, do, 0.43, causal)
        want = _torch_grads(q, k, v, do, 0.43, causal)
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            _close(g, w, tol=1e-12, what=f"{name} {B, H, Hkv, Nq, Nk, d, causal}")


def pin_bwd_finite_differences(orc):
    """Central differences of L = sum(dO * O) through the forward oracle (no backward code)."""
    rng = np.random.default_rng(31)
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 4, 6, 3
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, Nq, H, d))
    eps = 1e-5
    for causal in (False, True):
        grads = orc.attention_bwd(q, k, v, do, 0.8, causal)
        for which, x in enumerate((q, k, v)):
            for _ in range(6):
                idx = tuple(int(rng.integers(n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                lp = float(np.sum(do * orc.attention(*args_p, 0.8, causal)[0]))
                lm = float(np.sum(do * orc.attention(*args_m, 0.8, causal)[0]))
                fd = (lp - lm) / (2 * eps)
                g = grads[which][idx]
                assert abs(fd - g) <= 1e-7 * max(1.0, abs(g)), f"grad {which} {idx}: fd {fd} vs {g}"


def pin_bwd_invariants(orc):
    """Closed forms: per (batch, K/V head) the key gradients sum to zero (every row of dS
    sums to zero); the value gradients sum to the upstream rows that see a key; equal keys
    give dQ = 0; scale 0 gives dQ = dK = 0 and dV_j = sum of dO_i / (keys of row i)."""
    rng = np.random.default_rng(32)
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 6, 5, 3
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, Nq, H, d))
    G = H // Hkv
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.6, causal)
        _close(dk.sum(axis=1), np.zeros((B, Hkv, d)), tol=1e-12, what="sum dK")
        has_key = np.array([min(Nk, i + Nk - Nq + 1) > 0 if causal else True for i in range(Nq)])
        want = (do * has_key[None, :, None, None]).sum(axis=1).reshape(B, Hkv, G, d).sum(axis=2)
        _close(dv.sum(axis=1), want, tol=1e-12, what="sum dV")
        ke = np.broadcast_to(k[:, :1], k.shape).copy()
        dq_e, _, _ = orc.attention_bwd(q, ke, v, do, 0.6, causal)
        _close(dq_e, np.zeros_like(dq_e), tol=1e-12, what="equal keys dQ")
        dq0, dk0, dv0 = orc.attention_bwd(q, k, v, do, 0.0, causal)
        _close(dq0, np.zeros_like(dq0), what="scale 0 dQ")
        _close(dk0, np.zeros_like(dk0), what="scale 0 dK")
        nk = np.array([max(0, min(Nk, i + Nk - Nq + 1)) if causal else Nk for i in range(Nq)])
        want = np.zeros_like(dv0)
        for i in range(Nq):
            if nk[i]:
                contrib = do[:, i].reshape(B, Hkv, G, d).sum(axis=2) / nk[i]
                want[:, :nk[i]] += contrib[:, None]
        _close(dv0, want, tol=1e-12, what="scale 0 dV")


def pin_bwd_varlen_is_per_sequence(orc):
    """Packed varlen gradients equal separate calls on each sequence."""
    rng = np.random.default_rng(33)
    lengths = [3, 1, 6]
    H, Hkv, d = 4, 2, 3
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = off[-1]
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    do = rng.standard_normal((T, H, d))
    for causal in (False, True):
        got = orc.attention_bwd_varlen(q, k, v, do, off, 0.5, causal)
        for b in range(len(lengths)):
            sl = slice(off[b], off[b + 1])
            one = orc.attention_bwd(q[None, sl], k[None, sl], v[None, sl], do[None, sl], 0.5, causal)
            for name, g, w in zip(("dQ", "dK", "dV"), got, one):
                _close(g[sl], w[0], what=f"{name} seq {b}")


def pin_bwd_rows_torch_autograd(orc):
    """Selected gradient rows (one batch entry, one K/V head with its G query heads) vs
    torch's fp64 autograd of SDPA, including Nq != Nk, causal rows without keys and G > 1."""
    rng = np.random.default_rng(32)
    for (Nq, Nk, G, d, causal) in [(7, 7, 1, 4, True), (5, 9, 3, 6, True), (9, 4, 2, 5, True),
                                   (6, 8, 2, 3, False)]:
        q = rng.standard_normal((1, Nq, G, d))
        k = rng.standard_normal((1, Nk, 1, d))
        v = rng.standard_normal((1, Nk, 1, d))
        do = rng.standard_normal((1, Nq, G, d))
        want = _torch_grads(q, k, v, do, 0.61, causal)
        qrows = [(g, i) for g in range(G) for i in range(Nq)]
        krows = list(range(Nk))[::-1]
        dq, dk, dv = orc.attention_bwd_rows(q[0], k[0, :, 0], v[0, :, 0], do[0], 0.61, causal,
                                            qrows, krows)
        for r, (g, i) in enumerate(qrows):
            _close(dq[r], want[0][0, i, g], tol=1e-12, what=f"dQ row {(g, i)} {Nq, Nk, G, causal}")
        for r, j in enumerate(krows):
            _close(dk[r], want[1][0, j, 0], tol=1e-12, what=f"dK row {j} {Nq, Nk, G, causal}")
            _close(dv[r], want[2][0, j, 0], tol=1e-12, what=f"dV row {j} {Nq, Nk, G, causal}")


ALL_PINS = [pin_worked_example, pin_causal_figure12, pin_bottom_right_alignment,
            pin_exercise7_bounds, pin_torch_sdpa, pin_rows_sum_to_one, pin_shift_invariance,
            pin_causal_row0, pin_convex_hull, pin_future_independence, pin_scale_zero_mean,
            pin_rows_without_keys, pin_key_permutation, pin_head_batch_slices,
            pin_varlen_is_per_sequence, pin_rows_match_full, pin_torch_sdpa_grouped_heads,
            pin_gqa_exercise8, pin_gqa_equals_repeated_heads, pin_bwd_torch_autograd,
            pin_bwd_finite_differences, pin_bwd_invariants, pin_bwd_varlen_is_per_sequence,
            pin_bwd_rows_torch_autograd]
