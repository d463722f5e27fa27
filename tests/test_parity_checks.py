"""The comparisons the GPU parity tests rely on, checked on the CPU with known
answers: outputs equal to the oracle's (or its bf16 rounding) pass, and each
kind of error the bounds exist for fails -- one element past the element
bound, a shifted mean, a perturbed LSE, a changed -inf pattern, a NaN.  A
comparison that accepted everything would make every parity test vacuous."""
import numpy as np
import pytest

import oracle
from flashattention_forward_fa_amd import workloads as wl
from tests import parity


@pytest.fixture(scope="module")
def ref():
    w = wl.make_fixed(1, 2, 70, 90, 64, seed=17, causal=True)
    q, k, v = parity.inputs_f64(w)
    o, lse = oracle.attention(q, k, v, w.scale, w.causal)
    return o, lse


def _bf16(x):
    return wl.bf16_to_f64(wl.bf16_bits(np.asarray(x, dtype=np.float32)))


def test_exact_and_bf16_rounded_outputs_pass(ref):
    o, lse = ref
    parity.compare(o, lse, o, lse, bf16_out=False, what="exact")
    parity.compare(_bf16(o), lse.astype(np.float32), o, lse, bf16_out=True, what="bf16 O")


def test_one_element_past_the_bound_fails(ref):
    o, lse = ref
    bad = o.copy()
    bad[0, 5, 1, 3] += 1.5e-2
    with pytest.raises(AssertionError, match="O error"):
        parity.compare(bad, lse, o, lse, bf16_out=False)
    # with bf16 output the bar stays 1e-2 for every |O_ref| below 4 ...
    i = np.unravel_index(np.argmax(np.abs(o)), o.shape)
    assert abs(o[i]) < parity.BF16_ALLOWANCE_FROM
    bad = o.copy()
    bad[i] += parity.O_MAX_ABS * 1.01
    with pytest.raises(AssertionError, match="O error"):
        parity.compare(bad, lse, o, lse, bf16_out=True)


def test_bf16_allowance_only_from_four():
    """The representability allowance: 1e-2 below |O_ref| = 4 (where a bf16 half
    ulp is at most 2^-8 * 4 = 0.0078 < 1e-2), max(1e-2, half ulp + 1e-3) from 4
    on (0.0166 in [4, 8)); elements under it are counted."""
    o_ref = np.array([0.5, 1.5, 3.99, 4.0, 6.0, 9.0])
    b = parity.o_bound(o_ref, bf16_out=True)
    np.testing.assert_array_equal(b[:3], [1e-2, 1e-2, 1e-2])
    np.testing.assert_allclose(b[3:], [2.0 ** -6 + 1e-3, 2.0 ** -6 + 1e-3, 2.0 ** -5 + 1e-3])
    np.testing.assert_array_equal(parity.o_bound(o_ref, bf16_out=False), np.full(6, 1e-2))
    # (padded with exact elements so the mean bound is not what decides)
    o_ref = np.concatenate([o_ref, np.zeros(100)])
    lse = np.zeros(o_ref.size)
    # an error of 0.012 passes at 6.0 (allowance) and fails at 3.99 (plain bar)
    got = o_ref.copy()
    got[4] += 0.012
    st = parity.compare(got, lse, o_ref, lse, bf16_out=True)
    assert st["n_allowance"] == 3 and st["n_over_1e2"] == 1
    got = o_ref.copy()
    got[2] += 0.012
    with pytest.raises(AssertionError, match="O error"):
        parity.compare(got, lse, o_ref, lse, bf16_out=True)


def test_labelled_comparisons_are_recorded(ref):
    o, lse = ref
    n = len(parity.RECORDS)
    parity.compare(o, lse, o, lse, bf16_out=False, label="cpu check")
    assert len(parity.RECORDS) == n + 1
    label, st = parity.RECORDS.pop()
    assert label == "cpu check" and st["o_max_abs"] == 0.0 and st["n_elem"] == o.size
    assert st["lse_max_floor_rel"] == 0.0


def test_shifted_mean_fails(ref):
    o, lse = ref
    with pytest.raises(AssertionError, match="mean"):
        parity.compare(o + 2e-3, lse, o, lse, bf16_out=False)


def test_lse_errors_fail(ref):
    o, lse = ref
    bad = lse.copy()
    bad[0, 1, 10] += 2e-3 * max(1.0, abs(lse[0, 1, 10]))
    with pytest.raises(AssertionError, match="LSE error"):
        parity.compare(o, bad, o, lse, bf16_out=False)
    bad = lse.copy()
    bad[0, 0, 0] = -np.inf
    with pytest.raises(AssertionError, match="-inf pattern"):
        parity.compare(o, bad, o, lse, bf16_out=False)


def test_non_finite_output_fails(ref):
    o, lse = ref
    bad = o.copy()
    bad[0, 3, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        parity.compare(bad, lse, o, lse, bf16_out=False)


def test_gradient_bounds():
    rng = np.random.default_rng(18)
    r = [rng.standard_normal((40, 2, 16)) for _ in range(3)]
    rms = float(np.sqrt(np.mean(r[0] ** 2)))
    parity.compare_grads(r, r, "exact")
    # one element 0.1 rms off (the element bound is 2^-7 |R| + 0.05 rms)
    bad = [x.copy() for x in r]
    i = (3, 1, 4)
    bad[0][i] += 2.0 ** -7 * abs(r[0][i]) + 0.06 * rms
    with pytest.raises(AssertionError, match="dQ"):
        parity.compare_grads(bad, r, "one element")
    # ... which an allowance of that size admits at that element
    extra = np.zeros_like(r[0])
    extra[i] = 0.02 * rms
    parity.compare_grads(bad, r, "with allowance", extra=(extra, 0.0, 0.0))
    # a shifted mean fails even with every element inside its bound
    with pytest.raises(AssertionError):
        parity.compare_grads([r[0], r[1] + 0.004 * float(np.sqrt(np.mean(r[1] ** 2))), r[2]], r,
                             "mean")


def test_sampled_rows_cover_edges_and_stay_in_range():
    w = wl.make_fixed(2, 3, 300, 300, 64, seed=19, causal=True)
    rows = parity.sample_rows(w, 20, seed=1)
    assert rows[:, 0].max() < w.B and rows[:, 1].max() < w.H and rows[:, 2].max() < w.Nq
    assert rows.min() >= 0
    for i in (0, 127, 128, 255, 256, w.Nq - 1):
        assert i in set(rows[:, 2].tolist())
    wv = wl.make_varlen(2, 64, seed=20, lengths=[5, 0, 300])
    rv = parity.sample_rows(wv, 10, seed=2)
    for b, h, i in rv:
        assert 0 <= i < wv.lengths[b] and 0 <= h < wv.H
