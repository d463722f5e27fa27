"""HIP path vs the fp64 oracle, through the C ABI, element by element.

Small problems (several tiles, ragged tails, edge cases) are compared in full;
the five measured configurations run at their full sizes in the launch
configuration the benchmark times and are compared in full, every element of
O and LSE; the grouped-head variant of the headline workload is compared on
sampled rows (tile and block edges, first/last rows, random rows) that the
oracle computes one by one.
Both the conditional rescale (tau = 8) and the always-rescale variant (tau = 0)
must pass.
"""
import math

import numpy as np
import pytest

import oracle
from flashattention_forward_fa_amd import workloads as wl
from tests import parity
from tests.oracle_pins import load_worked_example

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_fa_amd as fa
    fa.load()   # raises if libfa.so is missing: there is no fallback


def _full_check(w, tau, o_dtype=None, what=""):
    o, lse = parity.run_gpu(w, tau=tau, o_dtype=o_dtype)
    q, k, v = parity.inputs_f64(w)
    if w.varlen:
        o_ref, lse_ref = oracle.attention_varlen(q, k, v, w.offsets, w.scale, w.causal)
    else:
        o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    bf16_out = (o_dtype == 0) if o_dtype is not None else (w.o_dtype == "bf16")
    return parity.compare(o, lse, o_ref, lse_ref, bf16_out=bf16_out, what=what or w.name)


# ------------------------------------------------------------ worked example

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("o_dtype", [0, 1])
def test_worked_example_padded(causal, o_dtype):
    """The page's 2-query / 4-key example with s = ln 2, zero-padded to d = 64 (exact in bf16).

    Non-causal: O = [[7/8, 3/4], [4/3, 1/3]], LSE = (ln 8, ln 9) as printed.
    Causal, bottom-right (Nq = 2, Nk = 4): O = [[5/7, 6/7], [4/3, 1/3]], LSE = (ln 7, ln 9).
    """
    import torch
    import flashattention_forward_fa_amd as fa
    g = load_worked_example()
    d = 64
    pad = lambda x: np.pad(x, ((0, 0), (0, d - x.shape[1])))
    mk = lambda x: torch.from_numpy(wl.bf16_bits(pad(x)[None, :, None, :].astype(np.float32))
                                    .view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = mk(g["Q"]), mk(g["K"]), mk(g["V"])
    for tau in (8.0, 0.0):
        o, lse = fa.attention(q, k, v, math.log(2.0), causal, o_dtype=o_dtype, rescale_threshold=tau)
        torch.cuda.synchronize()
        o = o.double().cpu().numpy()[0, :, 0, :2]
        lse = lse.double().cpu().numpy()[0, 0]
        if causal:
            want_o = [[5 / 7, 6 / 7], [4 / 3, 1 / 3]]
            want_l = [math.log(7), math.log(9)]
        else:
            want_o = [[7 / 8, 3 / 4], [4 / 3, 1 / 3]]
            want_l = [math.log(8), math.log(9)]
        tol = 1e-5 if o_dtype == 1 else 4e-3
        np.testing.assert_allclose(o, want_o, atol=tol)
        np.testing.assert_allclose(lse, want_l, atol=1e-5)


# ------------------------------------------------------------ small, full compare

SMALL = [
    # B, H, Nq, Nk, d, causal
    (2, 3, 300, 300, 64, False),
    (2, 3, 300, 300, 64, True),
    (1, 4, 300, 300, 128, False),
    (1, 4, 300, 300, 128, True),
    (1, 2, 100, 700, 128, True),     # Nq < Nk: bottom-right alignment
    (1, 2, 100, 700, 64, False),
    (1, 2, 700, 100, 128, True),     # Nq > Nk: leading rows have no key
    (2, 1, 1, 1, 64, True),
    (1, 3, 1, 1000, 128, True),
    (1, 2, 257, 513, 128, False),    # one past a tile / block boundary
    (3, 5, 64, 64, 128, True),
    (1, 8, 512, 512, 64, True),      # B*H a multiple of 8: XCD-aware order
]


@pytest.mark.parametrize("tau", [8.0, 0.0])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}q{}k{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_small_full(shape, tau):
    B, H, Nq, Nk, d, causal = shape
    w = wl.make_fixed(B, H, Nq, Nk, d, seed=B * 1000 + Nq + Nk + d, causal=causal)
    _full_check(w, tau)
    _full_check(w, tau, o_dtype=1, what=w.name + "/f32out")


@pytest.mark.parametrize("tau", [8.0, 0.0])
def test_small_outliers_force_rescale(tau):
    """K rows scaled by 8 (the long-sequence recipe) at a size the oracle finishes in full."""
    w = wl.make_fixed(1, 4, 1000, 1000, 128, seed=77, causal=True, outlier_frac=0.01)
    _full_check(w, tau)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.7])
def test_scale_values(scale):
    """Negative, zero and large scales (scale 0: O is the mean of the valid V rows)."""
    w = wl.make_fixed(1, 2, 200, 300, 64, seed=5, causal=True, scale=scale)
    _full_check(w, 8.0, o_dtype=1)


def _scaled_v(w, k, heads=None):
    """The workload with V multiplied by 2^k (exact in bf16), on every head or on `heads`."""
    import dataclasses
    v = wl.bf16_to_f32(w.v)
    if heads is None:
        v = v * np.float32(2.0 ** k)
    else:
        v[..., heads, :] *= np.float32(2.0 ** k)
    return dataclasses.replace(w, v=wl.bf16_bits(v))


@pytest.mark.parametrize("d", [64, 128])
def test_v_beyond_fp16_range(d):
    """V values of magnitude 2^16 and more have no fp16 value: such a tile is
    computed again with V staged as V * 2^-vk, and O scaled back.  Scaling V by
    2^20 must scale O by exactly 2^20 (fp32 and bf16 O), and the result must
    match the oracle relative to max |V|; heads whose V stays small are
    untouched by another head's rerun."""
    import dataclasses
    w = wl.make_fixed(1, 3, 300, 300, d, seed=88, causal=True)
    # no |v| below 2^-8: tiny values are fp16 subnormals unscaled but normal
    # scaled, which would round them differently
    v = wl.bf16_to_f32(w.v)
    v = np.where(np.abs(v) < 2.0 ** -8, np.copysign(np.float32(2.0 ** -8), v), v)
    w = dataclasses.replace(w, v=wl.bf16_bits(v.astype(np.float32)))
    big = _scaled_v(w, 20)
    for o_dtype in (1, 0):
        o0, l0 = parity.run_gpu(w, o_dtype=o_dtype)
        o1, l1 = parity.run_gpu(big, o_dtype=o_dtype)
        assert np.array_equal(o1, o0 * 2.0 ** 20), o_dtype
        assert np.array_equal(l1, l0)
    q, k, v = parity.inputs_f64(big)
    o_ref, lse_ref = oracle.attention(q, k, v, big.scale, big.causal)
    o1, l1 = parity.run_gpu(big, o_dtype=1)
    vmax = float(np.abs(v).max())
    assert np.abs(o1 - o_ref).max() <= 1e-2 * vmax / 4.0
    # one head's huge V: the other heads give what they give without it
    mixed = _scaled_v(w, 20, heads=[1])
    om, lm = parity.run_gpu(mixed, o_dtype=1)
    o0, l0 = parity.run_gpu(w, o_dtype=1)
    assert np.array_equal(om[:, :, [0, 2]], o0[:, :, [0, 2]])
    assert np.array_equal(om[:, :, 1], o0[:, :, 1] * 2.0 ** 20)


def test_tau_above_fp16_range_uses_bf16_p():
    """tau > 15 (P up to 2^tau would overflow fp16) rounds P to bf16: results
    still meet the bar in fp32 O, and tau = 15 (the largest fp16 threshold)
    too."""
    w = wl.make_fixed(1, 4, 500, 500, 128, seed=89, causal=True)
    for tau in (15.0, 16.0, 40.0):
        _full_check(w, tau, o_dtype=1, what=f"{w.name} tau={tau} f32 O")


def test_small_varlen_full():
    w = wl.make_varlen(3, 64, seed=31, nseq=5, len_lo=1, len_hi=700)
    _full_check(w, 8.0)
    _full_check(w, 0.0)
    w128 = wl.make_varlen(2, 128, seed=32, lengths=[300, 1, 256, 257, 40], causal=True)
    _full_check(w128, 8.0, o_dtype=1)
    wnc = wl.make_varlen(2, 64, seed=33, lengths=[17, 600, 129], causal=False)
    _full_check(wnc, 8.0)


def test_varlen_zero_length_sequences():
    """Sequences of length 0 inside a packed batch own no rows and no tiles."""
    w = wl.make_varlen(2, 128, seed=34, lengths=[5, 0, 130, 0, 64], causal=True)
    _full_check(w, 8.0)
    w64 = wl.make_varlen(3, 64, seed=35, lengths=[0, 257, 0], causal=False)
    _full_check(w64, 0.0, o_dtype=1)


def _xcd_order_lengths(seed):
    """70 sequence lengths in [0, 200) with two empty sequences and one of length 1:
    more than 64 sequences, so the per-wave scan over the offsets takes two rounds."""
    lengths = [int(x) for x in np.random.default_rng(seed).integers(0, 200, 70)]
    lengths[3] = lengths[64] = 0
    lengths[65] = 1
    return lengths


def test_varlen_xcd_order():
    """Head counts that are a multiple of 8 take the XCD-aware longest-first order
    (each XCD owns an eighth of the heads of every sequence, tiles of one head
    together): many and empty sequences, d = 64 and 128, grouped K/V heads."""
    w = wl.make_varlen(8, 64, seed=36, lengths=_xcd_order_lengths(36), causal=True)
    _full_check(w, 8.0)
    w128 = wl.make_varlen(16, 128, seed=37, lengths=[300, 0, 129, 513, 64], causal=True, Hkv=8)
    _full_check(w128, 8.0)


def test_varlen_many_short_sequences():
    """1000 sequences of 0 to 20 tokens (about 5% empty) with 8 heads: the XCD-aware
    order's scan over the offsets takes 16 rounds of 64 sequences."""
    lengths = [int(x) for x in np.random.default_rng(38).integers(0, 21, 1000)]
    w = wl.make_varlen(8, 64, seed=38, lengths=lengths, causal=True)
    _full_check(w, 8.0)
    wnc = wl.make_varlen(8, 128, seed=39, lengths=lengths[:300], causal=False)
    _full_check(wnc, 0.0)


def test_varlen_equals_separate_calls():
    """A packed call gives, bit for bit, what fixed-length calls on each sequence give."""
    w = wl.make_varlen(4, 128, seed=41, lengths=[513, 70, 256, 1000], causal=True)
    o, lse = parity.run_gpu(w)
    for b, L in enumerate(w.lengths):
        sl = slice(int(w.offsets[b]), int(w.offsets[b + 1]))
        one = wl.Workload("seq", 1, w.H, int(L), int(L), w.d, True, w.scale, "bf16", 0,
                          w.q[sl][None], w.k[sl][None], w.v[sl][None])
        o1, l1 = parity.run_gpu(one)
        assert np.array_equal(o[sl], o1[0]), f"sequence {b}"
        assert np.array_equal(lse[:, sl], l1[0]), f"sequence {b} lse"


def test_schedules_agree_bitwise():
    """Tile order changes which workgroup computes a tile, never its arithmetic."""
    # 16 (batch, head) pairs: two per XCD; 64: eight per XCD, in two head groups
    for H in (8, 32):
        w = wl.make_fixed(2, H, 600, 600, 128, seed=3, causal=True)
        t = parity.to_device(w)
        ref = parity.run_gpu(w, schedule=0, tensors=t)
        for sch in (1, 2):
            got = parity.run_gpu(w, schedule=sch, tensors=t)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (H, sch)
    wv = wl.make_varlen(3, 64, seed=4, lengths=[900, 10, 300, 513], causal=True)
    tv = parity.to_device(wv)
    ref = parity.run_gpu(wv, schedule=2, tensors=tv)
    got = parity.run_gpu(wv, schedule=1, tensors=tv)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    # 8 heads: the longest-first order of packed sequences is the XCD-aware one,
    # and it is the default for packed sequences with or without causal masking
    for causal in (False, True):
        wx = wl.make_varlen(8, 128, seed=6, lengths=[700, 0, 129, 64, 300], causal=causal)
        tx = parity.to_device(wx)
        ref = parity.run_gpu(wx, schedule=1, tensors=tx)
        for sch in (0, 2):
            got = parity.run_gpu(wx, schedule=sch, tensors=tx)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (causal, sch)


def test_outputs_stay_in_bounds():
    """Canary words around O and LSE are untouched (the kernel writes only its rows)."""
    import torch
    import flashattention_forward_fa_amd as fa
    w = wl.make_fixed(1, 3, 333, 333, 64, seed=9, causal=True)
    q, k, v, _ = parity.to_device(w)
    n_o = q.numel()
    pad = 256
    o_buf = torch.full((n_o + 2 * pad,), -12345.0, dtype=torch.float32, device="cuda")
    l_buf = torch.full((w.H * w.Nq + 2 * pad,), -777.0, dtype=torch.float32, device="cuda")
    o = o_buf[pad:pad + n_o]
    lse = l_buf[pad:pad + w.H * w.Nq]
    opts = fa.fa_fwd_opts_default()
    opts.o_dtype = fa.FA_DTYPE_F32
    st = fa.fa_fwd_ex(q, k, v, o, lse, 1, w.H, w.Nq, w.Nk, w.d, w.scale, 1, None, None, opts)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    ob = o_buf.cpu().numpy()
    lb = l_buf.cpu().numpy()
    assert np.all(ob[:pad] == -12345.0) and np.all(ob[pad + n_o:] == -12345.0)
    assert np.all(lb[:pad] == -777.0) and np.all(lb[pad + w.H * w.Nq:] == -777.0)
    assert np.all(np.isfinite(ob[pad:pad + n_o]))


# ------------------------------------------------------------ grouped K/V heads

GROUPED = [
    # B, H, Hkv, Nq, Nk, d, causal
    (2, 8, 2, 300, 300, 128, True),
    (1, 6, 3, 200, 333, 64, False),
    (1, 4, 1, 257, 257, 128, True),    # one K/V head (multi-query)
    (2, 8, 4, 100, 700, 64, True),     # Nq < Nk
]


@pytest.mark.parametrize("tau", [8.0, 0.0])
@pytest.mark.parametrize("shape", GROUPED, ids=lambda s: "B{}H{}kv{}q{}k{}d{}{}".format(*s[:6], "c" if s[6] else "f"))
def test_grouped_heads_full(shape, tau):
    B, H, Hkv, Nq, Nk, d, causal = shape
    w = wl.make_fixed(B, H, Nq, Nk, d, seed=H * 100 + Hkv + Nq, causal=causal, Hkv=Hkv)
    _full_check(w, tau)
    _full_check(w, tau, o_dtype=1, what=w.name + "/f32out")


def test_grouped_heads_varlen():
    w = wl.make_varlen(8, 64, seed=51, lengths=[300, 1, 129, 513], causal=True, Hkv=2)
    _full_check(w, 8.0)
    _full_check(w, 0.0)
    w = wl.make_varlen(4, 128, seed=52, lengths=[77, 256], causal=False, Hkv=1)
    _full_check(w, 8.0, o_dtype=1)


def test_grouped_equals_repeated_heads():
    """Grouped K/V heads give, bit for bit, what the same call gives on K/V with
    each head repeated G times consecutively (fixed length and varlen)."""
    import torch
    import flashattention_forward_fa_amd as fa
    for w in (wl.make_fixed(2, 8, 333, 333, 128, seed=53, causal=True, Hkv=2),
              wl.make_varlen(6, 64, seed=54, lengths=[200, 513, 3], causal=True, Hkv=3)):
        q, k, v, off = parity.to_device(w)
        G = w.H // w.kv_heads
        ax = 1 if w.varlen else 2
        kr = k.repeat_interleave(G, dim=ax).contiguous()
        vr = v.repeat_interleave(G, dim=ax).contiguous()
        ms = w.Nq if w.varlen else None
        o1, l1 = fa.attention(q, k, v, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
        o2, l2 = fa.attention(q, kr, vr, w.scale, w.causal, varlen_offsets=off, max_seqlen=ms)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), w.name


@pytest.mark.parametrize("tau", [8.0, 0.0])
def test_grouped_full_size(tau):
    """The causal B=2, H=32, N=4096, d=128 workload with 8 K/V heads, sampled rows."""
    w = wl.grouped(3, 8)
    rows = parity.sample_rows(w, n_random=256, seed=77)
    q, k, v = parity.inputs_f64(w)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, w.scale, w.causal, rows)
    del q, k, v
    o, lse = parity.run_gpu(w, tau=tau)
    go, gl = parity.gather_rows(w, o, lse, rows)
    label = f"{w.name} tau={tau:g} bf16 O, {len(rows)} rows"
    stats = parity.compare(go, gl, o_ref, lse_ref, bf16_out=True, what=label, label=label)
    print(f"{label}: {stats}")


# ------------------------------------------------------------ the five configurations

_REFS = {}


def _config_reference(n):
    """The fp64 oracle's O and LSE of configuration n over the whole workload,
    computed once per session (the default-path and the split-exp2 tests of a
    configuration compare against the same reference)."""
    if n not in _REFS:
        w = wl.config(n)
        q, k, v = parity.inputs_f64(w)
        if w.varlen:
            _REFS[n] = oracle.attention_varlen(q, k, v, w.offsets, w.scale, w.causal)
        else:
            _REFS[n] = oracle.attention(q, k, v, w.scale, w.causal)
    return _REFS[n]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_config(n):
    """Every element of O and LSE of the five measured workloads, at full size in
    the launch the benchmark times, against the fp64 oracle on the whole
    workload: both thresholds (tau = 8 conditional, tau = 0 always), each with
    the workload's O type and the other one (fp32 O holds the arithmetic to the
    plain bar; bf16 O is what the benchmark times)."""
    w = wl.config(n)
    o_ref, lse_ref = _config_reference(n)
    t = parity.to_device(w)
    own = 1 if w.o_dtype == "f32" else 0
    for tau in (8.0, 0.0):
        for o_dtype in (own, 1 - own):
            name = "f32" if o_dtype == 1 else "bf16"
            label = f"config {n} {w.name} tau={tau:g} {name} O"
            print(label, flush=True)
            o, lse = parity.run_gpu(w, tau=tau, tensors=t, o_dtype=o_dtype)
            stats = parity.compare(o, lse, o_ref, lse_ref, bf16_out=(o_dtype == 0), what=label,
                                   label=label)
            print(f"{label}: {stats}", flush=True)
            # properties over every row: LSE finite; causal row 0 is exactly V row 0
            assert np.all(np.isfinite(lse))
            if w.causal:
                v0 = wl.bf16_to_f64(w.v)
                if w.varlen:
                    first = w.offsets[:-1].astype(np.int64)
                    first = first[w.lengths > 0]
                    assert np.array_equal(o[first], v0[first])
                else:
                    assert np.array_equal(o[:, 0], v0[:, 0])
            del o, lse


# ------------------------------------------------------------ split exp2 (opt-in)

@pytest.mark.parametrize("n", [3, 5])
def test_exp2_poly_configs(n):
    """Half of the exponentials by the FMA polynomial (fa_fwd_opts.exp2_poly = 8):
    every element of the headline (d = 128) and the packed (d = 64) workloads,
    both thresholds, bf16 O, at the same bar as the default path."""
    w = wl.config(n)
    o_ref, lse_ref = _config_reference(n)
    t = parity.to_device(w)
    for tau in (8.0, 0.0):
        label = f"config {n} {w.name} tau={tau:g} bf16 O, exp2 poly 8/16"
        o, lse = parity.run_gpu(w, tau=tau, tensors=t, exp2_poly=8)
        stats = parity.compare(o, lse, o_ref, lse_ref, bf16_out=True, what=label, label=label)
        print(f"{label}: {stats}", flush=True)


@pytest.mark.parametrize("shape", SMALL[:8], ids=lambda s: "B{}H{}q{}k{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_exp2_poly_small(shape):
    """Ragged tails, Nq != Nk, rows without keys (P of masked keys exactly 0 on
    the polynomial path too), for each share of polynomial exponentials."""
    B, H, Nq, Nk, d, causal = shape
    w = wl.make_fixed(B, H, Nq, Nk, d, seed=B * 1000 + Nq + Nk + d + 7, causal=causal)
    q, k, v = parity.inputs_f64(w)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    for ep in (4, 8, 16):
        o, lse = parity.run_gpu(w, exp2_poly=ep)
        parity.compare(o, lse, o_ref, lse_ref, bf16_out=True, what=f"{w.name} exp2 poly {ep}/16")
