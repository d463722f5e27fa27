"""Backward pass (fa_bwd) vs the fp64 oracle, through the C ABI.

The GPU gets the forward's own outputs (O in bf16, LSE) and an upstream
gradient dO; the oracle recomputes everything in fp64 from Q, K, V and dO.
Bound, per gradient tensor G (dQ, dK, dV) with reference R, element-wise:

    |G - R| <= 2^-7 |R| + 0.05 * rms(R) + 1e-5,   mean |G - R| <= 3e-3 * rms(R)

Where the error comes from: the products that form the gradients take bf16
operands (P and dS rounded, 2^-9 relative each, independent over the summed
terms) and the result is rounded to bf16 (2^-9 relative) -- the 2^-7 |R| part.
D_i = rowsum(dO_i * O_i) uses O as the forward returns it, in bf16, so
D_i carries an error up to 2^-9 sum_c |dO_ic O_ic|; it shifts every dS_ij of
the row by P_ij times that error and so dQ_i by s * dD_i * sum_j P_ij k_j.  On
short causal rows (a handful of keys, P near 1) that term reaches a few
percent of the typical gradient size, hence the rms part.  The 1e-5 floor is
for gradients that are exactly zero (a row with one key has dS = 0; the GPU
gets dP - D rounded, about 1e-7).  Measured over these tests: the mean error
is 0.001-0.002 * rms(R), the bf16 rounding of the output; the largest errors,
up to 0.2 * rms(R), sit on large elements, within 2^-7 of their value.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_fa_amd import workloads as wl
from tests import parity
from tests.parity import compare_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_fa_amd as fa
    fa.load()


def run_bwd(w, dout_bits):
    import torch
    import flashattention_forward_fa_amd as fa
    q, k, v, off = parity.to_device(w)
    ms = w.Nq if w.varlen else None
    o, lse = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
    do = torch.from_numpy(dout_bits.view(np.int16)).view(torch.bfloat16).cuda()
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, w.scale, w.causal,
                                  varlen_offsets=off, max_seqlen=ms)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in (dq, dk, dv))


def ref_bwd(w, dout_bits):
    q, k, v = parity.inputs_f64(w)
    do = wl.bf16_to_f64(dout_bits)
    if w.varlen:
        return oracle.attention_bwd_varlen(q, k, v, do, w.offsets, w.scale, w.causal)
    return oracle.attention_bwd(q, k, v, do, w.scale, w.causal)


SHAPES = [
    # B, H, Hkv, Nq, Nk, d, causal
    (1, 2, 2, 100, 100, 64, False),
    (2, 3, 3, 300, 300, 64, True),
    (1, 4, 4, 257, 257, 128, True),
    (1, 2, 2, 64, 64, 128, False),
    (1, 2, 2, 100, 300, 128, True),     # Nq < Nk
    (1, 2, 2, 300, 100, 128, True),     # Nq > Nk: leading rows have no key
    (2, 4, 2, 200, 200, 128, True),     # grouped K/V heads
    (1, 4, 1, 129, 129, 64, False),     # one K/V head
    (2, 1, 1, 1, 1, 64, True),
    (1, 2, 2, 1, 500, 128, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}kv{}q{}k{}d{}{}".format(*s[:6], "c" if s[6] else "f"))
def test_bwd_small(shape):
    B, H, Hkv, Nq, Nk, d, causal = shape
    w = wl.make_fixed(B, H, Nq, Nk, d, seed=7000 + Nq + Nk + d + H, causal=causal, Hkv=Hkv)
    do = wl.make_dout(w, seed=8000 + Nq)
    stats = compare_grads(run_bwd(w, do), ref_bwd(w, do), w.name)
    print(w.name, stats)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_bwd_scales(scale):
    w = wl.make_fixed(1, 2, 150, 200, 64, seed=71, causal=True, scale=scale)
    do = wl.make_dout(w, seed=72)
    compare_grads(run_bwd(w, do), ref_bwd(w, do), f"scale {scale}")


def test_bwd_varlen():
    w = wl.make_varlen(4, 64, seed=73, lengths=[300, 1, 129, 513], causal=True, Hkv=2)
    do = wl.make_dout(w, seed=74)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "varlen d64 causal"))
    w = wl.make_varlen(2, 128, seed=75, lengths=[77, 256], causal=False)
    do = wl.make_dout(w, seed=76)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "varlen d128 full"))
    # sequences of length 0 inside the batch
    w = wl.make_varlen(2, 128, seed=77, lengths=[5, 0, 130, 0, 64], causal=True)
    do = wl.make_dout(w, seed=78)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "varlen with empty sequences"))


def row_term_allowance(q, k, v, do, scale, causal):
    """Four-sigma allowances for the D_i row term (derivation in
    test_bwd_full_size_sampled) on every row of one (sequence, K/V head) slice:
    q, do [Nq, G, d]; k, v [Nk, d].  Returns (dQ allowance [Nq, G, d], dK
    allowance [Nk, d])."""
    Nq, G, d = q.shape
    Nk = k.shape[0]
    o, lse = oracle.attention(q[None], k[None, :, None], v[None, :, None], scale, causal)
    kbar, _ = oracle.attention(q[None], k[None, :, None], k[None, :, None], scale, causal)
    sig = np.sqrt(np.sum((do * (2.0 ** -9 * np.abs(o[0]) + 3e-4)) ** 2, axis=2))     # [Nq, G]
    allow_q = abs(scale) * 4.0 * sig[:, :, None] * np.abs(kbar[0])
    sc = scale * np.einsum("igc,jc->igj", q, k)
    seen = np.ones((Nq, Nk), dtype=bool)
    if causal:
        seen = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
    lse_t = lse[0].T[:, :, None]
    pr = np.where(seen[:, None, :], np.exp(np.where(seen[:, None, :], sc - lse_t, -np.inf)), 0.0)
    allow_k = 4.0 * abs(scale) * np.sqrt(np.einsum("igj,igc->jc", (pr * sig[:, :, None]) ** 2, q ** 2))
    return allow_q, allow_k


def varlen_allowances(w, dout_bits):
    """row_term_allowance over every sequence and K/V head of a packed workload:
    ([T, H, d], [T, Hkv, d])."""
    q, k, v = parity.inputs_f64(w)
    do = wl.bf16_to_f64(dout_bits)
    G = w.H // w.kv_heads
    aq = np.zeros(q.shape)
    ak = np.zeros(k.shape)
    for b in range(len(w.lengths)):
        t = slice(int(w.offsets[b]), int(w.offsets[b + 1]))
        if t.stop == t.start:
            continue
        for kvh in range(w.kv_heads):
            hs = slice(kvh * G, (kvh + 1) * G)
            aq[t, hs], ak[t, kvh] = row_term_allowance(q[t, hs], k[t, kvh], v[t, kvh], do[t, hs],
                                                       w.scale, w.causal)
    return aq, ak


def test_bwd_varlen_xcd_order():
    """Head counts that are a multiple of 8 take the XCD-aware varlen order in both
    kernels: more than 64 sequences (two scan rounds) with empty ones; 16 query
    heads over 8 K/V heads.  Most rows here are short causal rows, where one key
    can dominate, so dQ and dK carry the D_i row-term allowance of the full-size
    checks."""
    lengths = [int(x) for x in np.random.default_rng(79).integers(0, 200, 70)]
    lengths[3] = lengths[64] = 0
    lengths[65] = 1
    w = wl.make_varlen(8, 64, seed=79, lengths=lengths, causal=True)
    do = wl.make_dout(w, seed=80)
    aq, ak = varlen_allowances(w, do)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "varlen 70 sequences H8",
                        extra=(aq, ak, 0.0)))
    w = wl.make_varlen(16, 128, seed=81, lengths=[300, 0, 129, 513, 64], causal=True, Hkv=8)
    do = wl.make_dout(w, seed=82)
    aq, ak = varlen_allowances(w, do)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "varlen H16 over 8 K/V heads",
                        extra=(aq, ak, 0.0)))


def test_bwd_varlen_many_short_sequences():
    """1000 sequences of 0 to 20 tokens with 8 heads (16 scan rounds in both kernels)."""
    lengths = [int(x) for x in np.random.default_rng(83).integers(0, 21, 1000)]
    w = wl.make_varlen(8, 64, seed=83, lengths=lengths, causal=True)
    do = wl.make_dout(w, seed=84)
    aq, ak = varlen_allowances(w, do)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), "1000 short sequences H8",
                        extra=(aq, ak, 0.0)))


def test_bwd_mid_size():
    """Many key and query blocks: B=1, H=4, N=1024, d=128, causal."""
    w = wl.make_fixed(1, 4, 1024, 1024, 128, seed=77, causal=True)
    do = wl.make_dout(w, seed=78)
    print(compare_grads(run_bwd(w, do), ref_bwd(w, do), w.name))


def test_bwd_deterministic():
    """Two calls give the same bits (no atomics, fixed reduction order)."""
    w = wl.make_fixed(2, 4, 333, 333, 128, seed=79, causal=True, Hkv=2)
    do = wl.make_dout(w, seed=80)
    a = run_bwd(w, do)
    b = run_bwd(w, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _sample(n, rng, count, block=128):
    """Row indices: first/last, the edges of every 128-row tile (capped), and random rows."""
    edges = sorted({0, n - 1} | {x for t in range(0, n, block) for x in (t, t + block - 1) if x < n})
    if len(edges) > 48:
        edges = edges[:24] + edges[-24:]
    extra = rng.integers(0, n, count) if n > 0 else np.zeros(0, dtype=np.int64)
    return sorted(set(edges) | {int(x) for x in extra})


FULL_SIZE = ["2", "3", "4", "5", "3-kv8"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_bwd_full_size_sampled(name):
    """The measured workloads at full size, in the launch the benchmark times
    (fa_bwd on the forward's O and LSE, dO from seed + 500); the oracle computes
    sampled dQ rows and dK, dV rows of two (batch or sequence, K/V head) slices.

    Row-term allowance for dQ.  The GPU forms D_i = dO_i . O_i from the
    forward's bf16 O, whose elements differ from the exact O by their bf16
    rounding (up to 2^-9 |O|) plus the forward's own error (mean 2.6e-4,
    measured); an error dD_i moves every dS_ij of the row by -P_ij dD_i and so
    dQ_i by -scale dD_i Kbar_i with Kbar_i = sum_j P_ij k_j.  The d per-element
    errors are independent, so dD_i is taken at four standard deviations of
    their sum, 4 sqrt(sum_c dO_ic^2 (2^-9 |O_ic| + 3e-4)^2), and the allowance
    for element (i, c) is scale dD_i |Kbar_ic|; O_i and Kbar_i come from the
    oracle's forward (Kbar_i is attention with V := K).  It matters where one
    key dominates a row and that key is large: the outlier keys of the
    N = 16384 workload (8x scaled rows) make Kbar large exactly there.

    The same errors reach dK_j = scale sum_i dS_ij q_i as -scale sum_i P_ij dD_i
    q_i, a sum of independent terms over the queries (of all G heads) that see
    key j; its allowance is four standard deviations,
    4 scale sqrt(sum_i P_ij^2 sigma_i^2 q_ic^2) with sigma_i the one-sigma dD_i
    above, and P_ij = exp(scale q_i.k_j - LSE_i) from the oracle's LSE.  It
    matters for the first keys of a causal sequence, which every query sees
    and which carry most of the weight of the short rows."""
    w = wl.grouped(3, 8) if name == "3-kv8" else wl.config(int(name))
    dout = wl.make_dout(w, seed=w.seed + 500)
    dq, dk, dv = run_bwd(w, dout)
    G = w.H // w.kv_heads
    rng = np.random.default_rng(4242 + len(name))
    if w.varlen:
        order = np.argsort(w.lengths)
        slices = [(int(order[-1]), 0), (int(order[len(order) // 2]), w.kv_heads - 1)]
    else:
        slices = [(0, 0), (w.B - 1, w.kv_heads - 1)]
    for (b, kvh) in slices:
        hs = slice(kvh * G, (kvh + 1) * G)
        if w.varlen:
            t = slice(int(w.offsets[b]), int(w.offsets[b + 1]))
            sel = lambda x, hsl: x[t, hsl]
        else:
            sel = lambda x, hsl: x[b, :, hsl]
        q = wl.bf16_to_f64(sel(w.q, hs))
        k = wl.bf16_to_f64(sel(w.k, kvh))
        v = wl.bf16_to_f64(sel(w.v, kvh))
        do = wl.bf16_to_f64(sel(dout, hs))
        Nq, Nk = q.shape[0], k.shape[0]
        qi = _sample(Nq, rng, 48)
        qrows = [(g, i) for i in qi for g in range(G)]
        krows = _sample(Nk, rng, 48)
        rq, rk, rv = oracle.attention_bwd_rows(q, k, v, do, w.scale, w.causal, qrows, krows)
        rows3 = [(0, g, i) for (g, i) in qrows]
        o_ref, _ = oracle.attention_rows(q[None], k[None, :, None], v[None, :, None], w.scale,
                                         w.causal, rows3)
        kbar, _ = oracle.attention_rows(q[None], k[None, :, None], k[None, :, None], w.scale,
                                        w.causal, rows3)
        do_rows = np.stack([do[i, g] for (g, i) in qrows])
        dD = 4.0 * np.sqrt(np.sum((do_rows * (2.0 ** -9 * np.abs(o_ref) + 3e-4)) ** 2, axis=1))
        allow_q = abs(w.scale) * dD[:, None] * np.abs(kbar)
        o_all, lse_all = oracle.attention(q[None], k[None, :, None], v[None, :, None], w.scale,
                                          w.causal)
        sig = np.sqrt(np.sum((do * (2.0 ** -9 * np.abs(o_all[0]) + 3e-4)) ** 2, axis=2))  # [Nq,G]
        kr = np.asarray(krows)
        sc = w.scale * np.einsum("igc,jc->igj", q, k[kr])
        seen = np.ones((Nq, kr.size), dtype=bool)
        if w.causal:
            seen = kr[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        lse_t = lse_all[0].T[:, :, None]                                    # [Nq,G,1]
        pr = np.where(seen[:, None, :], np.exp(np.where(seen[:, None, :], sc - lse_t, -np.inf)), 0.0)
        allow_k = 4.0 * abs(w.scale) * np.sqrt(np.einsum("igj,igc->jc", (pr * sig[:, :, None]) ** 2,
                                                         q ** 2))
        gq = np.stack([sel(dq, hs)[i, g] for (g, i) in qrows])
        gk = np.stack([sel(dk, kvh)[j] for j in krows])
        gv = np.stack([sel(dv, kvh)[j] for j in krows])
        stats = compare_grads((gq, gk, gv), (rq, rk, rv), f"{w.name} slice {(b, kvh)}",
                              extra=(allow_q, allow_k, 0.0))
        stats["dQ"]["mean_allowance_over_rms"] = float(0.25 * allow_q.mean() / stats["dQ"]["rms"])
        print(w.name, (b, kvh), stats)
