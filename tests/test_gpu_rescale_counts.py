"""Rescale decisions of the forward kernel against the blockwise model.

O and LSE do not depend on when the exponent reference moves (any consistent
reference gives the same result), so the output parity tests cannot see the
decision logic.  With ``fa_fwd_opts.rescale_counts`` the kernel writes, per
query row, how many K/V blocks after the row's first one moved its reference
("Flash Attention 4", section "algorithm structure": delta < -tau).  The
blockwise fp64 model (oracle/model.py) walks the same 64-key blocks in the same
order and counts the same events.  The counts must be equal on every row
whose decisions are not near ties (|delta + tau| < 1e-3 on some block, where
the kernel's fp32 scores may decide the other way); on those rows they may
differ by at most the number of near ties.  Integer work: exact elsewhere.
"""
import numpy as np
import pytest

from flashattention_forward_fa_amd import workloads as wl
from oracle import model
from tests import parity

pytestmark = pytest.mark.gpu
BLOCK_N = 64   # the kernel's K/V block


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_fa_amd as fa
    fa.load()


def gpu_counts(w, tau):
    import torch
    import flashattention_forward_fa_amd as fa
    q, k, v, off = parity.to_device(w)
    ms = w.Nq if w.varlen else None
    o, lse, cnt = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms,
                               rescale_threshold=tau, rescale_counts=True)
    o2, lse2 = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms,
                            rescale_threshold=tau)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "counting changed the outputs"
    return cnt.cpu().numpy()


def check_slices(w, tau, cnt, slices):
    """slices: (b, h) pairs; cnt laid out like lse."""
    G = w.H // w.kv_heads
    total = 0
    for (b, h) in slices:
        if w.varlen:
            t = slice(int(w.offsets[b]), int(w.offsets[b + 1]))
            q = wl.bf16_to_f64(w.q[t, h])
            k = wl.bf16_to_f64(w.k[t, h // G])
            v = wl.bf16_to_f64(w.v[t, h // G])
            got = cnt[h, t]
        else:
            q = wl.bf16_to_f64(w.q[b, :, h])
            k = wl.bf16_to_f64(w.k[b, :, h // G])
            v = wl.bf16_to_f64(w.v[b, :, h // G])
            got = cnt[b, h]
        r = model.fa4_forward(q, k, v, w.scale, causal=w.causal, block_n=BLOCK_N, threshold=tau)
        want, ties = r["rescale_rows"], r["near_ties"]
        diff = np.abs(got.astype(np.int64) - want)
        clean = ties == 0
        bad = np.nonzero(clean & (diff != 0))[0]
        assert bad.size == 0, (f"{w.name} tau={tau} slice {(b, h)}: rows {bad[:8].tolist()} "
                               f"gpu {got[bad[:8]].tolist()} model {want[bad[:8]].tolist()}")
        assert np.all(diff <= ties), f"{w.name} tau={tau} slice {(b, h)}: near-tie rows off by more"
        total += int(want.sum())
    return total


SMALL = [
    # B, H, Hkv, Nq, Nk, d, causal, outlier fraction
    (1, 2, 2, 300, 300, 128, True, 0.02),
    (1, 2, 2, 257, 257, 64, True, 0.02),
    (2, 3, 3, 200, 333, 128, False, 0.03),
    (1, 2, 2, 100, 300, 128, True, 0.05),    # Nq < Nk
    (1, 2, 2, 300, 100, 64, True, 0.05),     # Nq > Nk: leading rows have no key
    (1, 4, 2, 500, 500, 128, True, 0.01),    # grouped K/V heads
]


@pytest.mark.parametrize("tau", [8.0, 0.0])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}kv{}q{}k{}d{}{}".format(*s[:6], "c" if s[6] else "f"))
def test_counts_small(shape, tau):
    B, H, Hkv, Nq, Nk, d, causal, frac = shape
    w = wl.make_fixed(B, H, Nq, Nk, d, seed=9000 + Nq + Nk + d, causal=causal, Hkv=Hkv,
                      outlier_frac=frac)
    cnt = gpu_counts(w, tau)
    total = check_slices(w, tau, cnt, [(b, h) for b in range(B) for h in range(H)])
    if tau == 0.0:
        assert total > 0


def test_counts_varlen():
    w = wl.make_varlen(2, 64, seed=91, lengths=[300, 1, 129, 513], causal=True)
    for tau in (8.0, 0.0):
        cnt = gpu_counts(w, tau)
        check_slices(w, tau, cnt, [(b, h) for b in range(4) for h in range(2)])


@pytest.mark.parametrize("n", [3, 4])
def test_counts_full_size(n):
    """The measured causal workloads at full size; on the long one the outlier keys
    (1% of K rows scaled by 8) make the conditional rescale happen (counts > 0 with
    tau = 8, fewer than with tau = 0)."""
    w = wl.config(n)
    slices = [(0, 0), (w.B - 1, w.H - 1)] if n == 3 else [(0, 5)]
    t8 = check_slices(w, 8.0, gpu_counts(w, 8.0), slices)
    t0 = check_slices(w, 0.0, gpu_counts(w, 0.0), slices)
    print(w.name, "rescale events tau=8:", t8, "tau=0:", t0)
    assert t8 < t0
    if n == 4:
        assert t8 > 0
