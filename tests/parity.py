"""Helpers shared by the GPU parity tests: upload a workload, run the HIP path
through the C ABI, and compare with the oracle at the stated tolerances.

Tolerances (O compared widened to fp64 against the unrounded fp64 oracle):
  * max |O - O_ref| <= 1e-2 and mean |O - O_ref| <= 1e-3, for fp32 and for
    bf16 output alike.
  * One exception, counted and reported: a bf16 value with |O_ref| >= 4 is
    rounded by up to half a bf16 ulp of its binade (2^-6 = 0.0156 in [4, 8)),
    which alone exceeds 1e-2; such elements are held to
    max(1e-2, half_ulp_bf16(O_ref) + 1e-3) instead.  Below 4 the half ulp is
    at most 0.0078 and the plain bound applies.
  * LSE: |LSE - LSE_ref| <= 1e-3 * max(1, |LSE_ref|) (a relative bound with a
    floor, since short causal rows can have LSE near 0); -inf must match -inf.

Every comparison made with a ``label`` is recorded in ``RECORDS`` (max-abs,
mean-abs, elements over 1e-2, elements under the representability allowance,
LSE errors); the test session prints them at its end.
"""
from __future__ import annotations

import math

import numpy as np

from flashattention_forward_fa_amd import workloads as wl

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_REL = 1e-3
BF16_ALLOWANCE_FROM = 4.0   # |O_ref| from which a bf16 element's half ulp exceeds the bar

RECORDS: list = []          # (label, stats) of every labelled comparison, in order


def to_device(w):
    import torch
    dev = "cuda"
    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.from_numpy(w.k.view(np.int16)).view(torch.bfloat16).to(dev)
    v = torch.from_numpy(w.v.view(np.int16)).view(torch.bfloat16).to(dev)
    off = None
    if w.varlen:
        off = torch.from_numpy(np.ascontiguousarray(w.offsets.astype(np.int32))).to(dev)
    return q, k, v, off


def run_gpu(w, *, tau=8.0, o_dtype=None, schedule=0, tensors=None, exp2_poly=0):
    """Run the HIP path on workload w; returns (o float64 numpy, lse float64 numpy)."""
    import torch
    import flashattention_forward_fa_amd as fa
    q, k, v, off = tensors if tensors is not None else to_device(w)
    if o_dtype is None:
        o_dtype = fa.FA_DTYPE_F32 if w.o_dtype == "f32" else fa.FA_DTYPE_BF16
    o, lse = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off,
                          max_seqlen=w.Nq if w.varlen else None, o_dtype=o_dtype,
                          rescale_threshold=tau, schedule=schedule, exp2_poly=exp2_poly)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def inputs_f64(w):
    return wl.bf16_to_f64(w.q), wl.bf16_to_f64(w.k), wl.bf16_to_f64(w.v)


def half_ulp_bf16(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def o_bound(o_ref, bf16_out: bool):
    """Per-element bound on |O - O_ref|: 1e-2, except bf16 elements with
    |O_ref| >= 4, which get max(1e-2, half_ulp_bf16(O_ref) + 1e-3)."""
    bound = np.full(np.shape(o_ref), O_MAX_ABS)
    if bf16_out:
        big = np.abs(o_ref) >= BF16_ALLOWANCE_FROM
        if big.any():
            bound[big] = np.maximum(O_MAX_ABS, half_ulp_bf16(o_ref[big]) + 1e-3)
    return bound


def compare(o, lse, o_ref, lse_ref, *, bf16_out: bool, what: str = "", label: str | None = None):
    """Assert the tolerances; returns a dict of error statistics (recorded in
    RECORDS under ``label`` when one is given, also when an assertion fails)."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o.shape == o_ref.shape, f"{what}: O shape {o.shape} vs {o_ref.shape}"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err = np.abs(o - o_ref)
    bound = o_bound(o_ref, bf16_out)
    bad = err > bound
    stats = dict(n_elem=int(err.size), o_max_abs=float(err.max(initial=0.0)),
                 o_mean_abs=float(err.mean()) if err.size else 0.0,
                 n_over_1e2=int(np.count_nonzero(err > O_MAX_ABS)),
                 n_allowance=int(np.count_nonzero(bound > O_MAX_ABS)))
    if label is not None:
        RECORDS.append((label, stats))
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: O error {err[idx]:.3e} > bound {bound[idx]:.3e} at {idx} "
                             f"(ref {o_ref[idx]:.5f}, got {o[idx]:.5f}); {int(bad.sum())} elements")
    assert stats["o_mean_abs"] <= O_MEAN_ABS, f"{what}: mean |dO| {stats['o_mean_abs']:.3e}"

    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert lse.shape == lse_ref.shape, f"{what}: LSE shape {lse.shape} vs {lse_ref.shape}"
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf_ref), f"{what}: -inf pattern of LSE differs"
    fin = ~ninf_ref
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite LSE"
    dl = np.abs(lse[fin] - lse_ref[fin])
    lb = LSE_REL * np.maximum(1.0, np.abs(lse_ref[fin]))
    if dl.size:
        stats["lse_max_abs"] = float(dl.max())
        stats["lse_max_rel"] = float((dl / np.maximum(np.abs(lse_ref[fin]), 1e-30)).max())
        stats["lse_max_floor_rel"] = float((dl / np.maximum(1.0, np.abs(lse_ref[fin]))).max())
        if np.any(dl > lb):
            j = int(np.argmax(dl - lb))
            raise AssertionError(f"{what}: LSE error {dl[j]:.3e} > {lb[j]:.3e} (ref {lse_ref[fin][j]})")
    return stats


def sample_rows(w, n_random: int, seed: int = 0):
    """(b, h, i) triples: tile and block edges, first and last rows, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    if w.varlen:
        for b, L in enumerate(w.lengths):
            L = int(L)
            for i in sorted({0, 1, 2, 31, 32, 63, 64, 255, 256, L // 2, L - 2, L - 1}):
                if 0 <= i < L:
                    rows.append((b, int(rng.integers(w.H)), i))
        live = [b for b, L in enumerate(w.lengths) if int(L) > 0]   # empty sequences own no rows
        for _ in range(n_random if live else 0):
            b = live[int(rng.integers(len(live)))]
            rows.append((b, int(rng.integers(w.H)), int(rng.integers(int(w.lengths[b])))))
    else:
        edges = sorted({0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, 257, w.Nq // 2,
                        w.Nq - 2, w.Nq - 1})
        for b in range(w.B):
            for h in (0, w.H - 1):
                for i in edges:
                    if 0 <= i < w.Nq:
                        rows.append((b, h, i))
        for _ in range(n_random):
            rows.append((int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.Nq))))
    return np.array(sorted(set(rows)), dtype=np.int64)


def gather_rows(w, o, lse, rows):
    """Pick the sampled rows out of full GPU outputs."""
    if w.varlen:
        t = w.offsets[rows[:, 0]].astype(np.int64) + rows[:, 2]
        return o[t, rows[:, 1]], lse[rows[:, 1], t]
    return o[rows[:, 0], rows[:, 2], rows[:, 1]], lse[rows[:, 0], rows[:, 1], rows[:, 2]]


def flops_str(w):
    return f"{w.flops() / 1e9:.2f} GFLOP"


def ln(x):
    return math.log(x)


def compare_grads(got, ref, what, extra=(0.0, 0.0, 0.0)):
    """Backward parity: per gradient tensor G (dQ, dK, dV) with reference R,
    |G - R| <= 2^-7 |R| + 0.05 rms(R) + 1e-5 element-wise and mean |G - R| <=
    3e-3 rms(R) (derivation in tests/test_gpu_backward.py).  extra: per-gradient
    allowance at four standard deviations, added to the element bound, and at
    one (a quarter of it) to the mean bound -- the row-term allowance of the
    full-size dQ and dK checks; 0 elsewhere."""
    stats = {}
    for name, g, r, ex in zip(("dQ", "dK", "dV"), got, ref, extra):
        assert g.shape == r.shape, f"{what} {name} shape"
        assert np.all(np.isfinite(g)), f"{what} {name} not finite"
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        err = np.abs(g - r)
        ex = np.broadcast_to(np.asarray(ex, dtype=np.float64), r.shape)
        bound = 2.0 ** -7 * np.abs(r) + 0.05 * rms + 1e-5 + ex
        stats[name] = dict(max_err=float(err.max(initial=0.0)), rms=rms,
                           max_over_rms=float(err.max(initial=0.0) / rms) if rms else 0.0,
                           mean_over_rms=float(err.mean() / rms) if rms and err.size else 0.0)
        bad = err > bound
        if bad.any():
            idx = np.unravel_index(np.argmax(err - bound), err.shape)
            raise AssertionError(f"{what} {name}: error {err[idx]:.3e} > {bound[idx]:.3e} at {idx} "
                                 f"(ref {r[idx]:.4f}, got {g[idx]:.4f}, rms {rms:.3e}); "
                                 f"{int(bad.sum())} elements")
        if rms:
            assert err.mean() <= 3e-3 * rms + 0.25 * ex.mean(), \
                f"{what} {name}: mean error {err.mean():.3e} vs rms {rms:.3e} (+{0.25 * ex.mean():.3e})"
    return stats
