"""The blockwise fp64 model of the online-softmax update (conditional and
always-rescale) against the worked example's round states, exercise 1 of the
FA4 page, and the three-pass oracle (no GPU)."""
import math

import numpy as np
import pytest

import oracle
from oracle import model
from tests.oracle_pins import load_worked_example, _frac

TOL = 1e-12


def test_worked_example_rounds_always_rescale():
    """Threshold 0 reproduces the page's rounds: figures 5-9, table 1, figure 10."""
    g = load_worked_example()
    r = model.fa4_forward(g["Q"], g["K"], g["V"], math.log(2.0), block_n=2, threshold=0.0,
                          trace=True)
    r1, r2 = r["trace"]
    np.testing.assert_allclose(r1["row_max"], g["round1"]["m"], atol=TOL)
    np.testing.assert_allclose(r1["P"], _frac(g["round1"]["P"]), atol=TOL)
    np.testing.assert_allclose(r1["row_sum"], _frac(g["round1"]["l"]), atol=TOL)
    np.testing.assert_allclose(r1["O"], _frac(g["round1"]["O"]), atol=TOL)
    np.testing.assert_allclose(r2["row_max"], g["round2"]["m"], atol=TOL)
    np.testing.assert_allclose(r2["acc_scale"], _frac(g["round2"]["alpha"]), atol=TOL)
    np.testing.assert_allclose(r2["P"], _frac(g["round2"]["P"]), atol=TOL)
    np.testing.assert_allclose(r2["row_sum"], _frac(g["round2"]["l"]), atol=TOL)
    np.testing.assert_allclose(r2["O"], _frac(g["round2"]["O"]), atol=TOL)
    np.testing.assert_allclose(r["o"], _frac(g["final"]["O"]), atol=TOL)
    np.testing.assert_allclose(r["lse"], [math.log(8.0), math.log(9.0)], atol=TOL)
    assert r["rescales"] == 2


def test_worked_example_rounds_conditional():
    """Threshold 8: at the example's second K/V block delta = (1 - 2) * 1 = -1 >= -8, so the reference stays 1.

    Derived from the update rule: P^(2) = 2^(S - 1) = [[2, 1/2], [1, 2]],
    l = 3/2 + (5/2, 3) = (4, 9/2), O = O^(1) + P^(2) V_2 = [[7/2, 3], [6, 3/2]];
    the final O and LSE equal the always-rescale ones.
    """
    g = load_worked_example()
    r = model.fa4_forward(g["Q"], g["K"], g["V"], math.log(2.0), block_n=2, threshold=8.0,
                          trace=True)
    r2 = r["trace"][1]
    np.testing.assert_allclose(r2["row_max"], [1.0, 1.0], atol=TOL)
    np.testing.assert_allclose(r2["acc_scale"], [1.0, 1.0], atol=TOL)
    np.testing.assert_allclose(r2["P"], [[2.0, 0.5], [1.0, 2.0]], atol=TOL)
    np.testing.assert_allclose(r2["row_sum"], [4.0, 4.5], atol=TOL)
    np.testing.assert_allclose(r2["O"], [[3.5, 3.0], [6.0, 1.5]], atol=TOL)
    np.testing.assert_allclose(r["o"], _frac(g["final"]["O"]), atol=TOL)
    np.testing.assert_allclose(r["lse"], [math.log(8.0), math.log(9.0)], atol=TOL)
    assert r["rescales"] == 0


def test_exercise1_keep_reference():
    """FA4 page exercise 1, S = [5, 4]: candidate 5, delta -3 >= -8 -> keep 2, acc 1."""
    cand, delta, ref, acc, P, l, O = model.update_row(2.0, 3.0, [4.0, 6.0], [5.0, 4.0],
                                                      np.eye(2), 1.0, threshold=8.0)
    assert (cand, delta, ref, acc) == (5.0, -3.0, 2.0, 1.0)
    np.testing.assert_array_equal(P, [8.0, 4.0])
    assert l == 15.0
    np.testing.assert_array_equal(O, [12.0, 10.0])


def test_exercise1_switch_reference():
    """S = [11, 10]: candidate 11, delta -9 < -8 -> switch, acc 2^-9, l = 771/512."""
    cand, delta, ref, acc, P, l, O = model.update_row(2.0, 3.0, [4.0, 6.0], [11.0, 10.0],
                                                      np.eye(2), 1.0, threshold=8.0)
    assert (cand, delta, ref, acc) == (11.0, -9.0, 11.0, 2.0 ** -9)
    np.testing.assert_array_equal(P, [1.0, 0.5])
    assert l == 771.0 / 512.0
    np.testing.assert_array_equal(O, [516.0 / 512.0, 262.0 / 512.0])


def test_exercise1_always_rescale_same_ratio():
    """Threshold 0 on S = [5, 4] rescales by 2^-3 but O / l is unchanged: (0.8, 2/3)."""
    _, _, ref, acc, _, l, O = model.update_row(2.0, 3.0, [4.0, 6.0], [5.0, 4.0], np.eye(2),
                                               1.0, threshold=0.0)
    assert ref == 5.0 and acc == 0.125
    np.testing.assert_allclose(O / l, [0.8, 2.0 / 3.0], atol=TOL)


def test_threshold_tie_keeps_reference():
    """delta exactly -tau keeps the old reference (the test is delta >= -threshold)."""
    _, delta, ref, acc, _, _, _ = model.update_row(0.0, 1.0, [0.0], [8.0], [[1.0]], 1.0,
                                                   threshold=8.0)
    assert delta == -8.0 and ref == 0.0 and acc == 1.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("threshold", [0.0, 8.0])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("block_n,Nq,Nk", [(1, 7, 7), (3, 9, 13), (16, 40, 33), (4, 10, 6)])
def test_model_matches_oracle(causal, threshold, reverse, block_n, Nq, Nk):
    """The update is exact for any consistent reference: model == three-pass oracle."""
    rng = np.random.default_rng(100 + Nq + Nk + block_n)
    d = 8
    q = rng.standard_normal((Nq, d)) * 2.0
    k = rng.standard_normal((Nk, d)) * 2.0
    v = rng.standard_normal((Nk, d))
    scale = 1.0 / math.sqrt(d)
    r = model.fa4_forward(q, k, v, scale, causal=causal, block_n=block_n, threshold=threshold,
                          reverse=reverse)
    o, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None], scale, causal)
    np.testing.assert_allclose(r["o"], o[0, :, 0], atol=1e-12, rtol=1e-12)
    both_inf = np.isneginf(r["lse"]) & np.isneginf(lse[0, 0])
    np.testing.assert_allclose(np.where(both_inf, 0, r["lse"]), np.where(both_inf, 0, lse[0, 0]),
                               atol=1e-12, rtol=1e-12)


def test_outlier_keys_force_rescales():
    """K rows scaled by 8 make the row maximum jump: the conditional variant still rescales,
    but less often than the always variant."""
    rng = np.random.default_rng(5)
    N, d = 512, 64
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    k[rng.choice(N, 5, replace=False)] *= 8.0
    v = rng.standard_normal((N, d))
    r8 = model.fa4_forward(q, k, v, 1 / 8, causal=True, block_n=64, threshold=8.0)
    r0 = model.fa4_forward(q, k, v, 1 / 8, causal=True, block_n=64, threshold=0.0)
    assert 0 < r8["rescales"] < r0["rescales"]
    np.testing.assert_allclose(r8["o"], r0["o"], atol=1e-12)


def test_fully_masked_first_blocks_stay_finite():
    """Reverse order with small blocks: a row's first visited blocks can be fully masked
    (candidate -inf); the guard keeps the state zero and the result finite."""
    rng = np.random.default_rng(6)
    N, d = 12, 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    r = model.fa4_forward(q, k, v, 0.5, causal=True, block_n=2, threshold=8.0, reverse=True)
    assert np.all(np.isfinite(r["o"])) and np.all(np.isfinite(r["lse"]))
    o, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None], 0.5, True)
    np.testing.assert_allclose(r["o"], o[0, :, 0], atol=1e-12)


def test_rescale_counts_per_row_by_hand():
    """Per-row reference moves, one key per block, scale ln 2 (scale * log2 e is exactly
    1.0 in fp64, so delta is the score gap).  Scores of row 0: 0, 5, 9, 12, 30, 31; row 1
    (twice the query): 0, 10, 18, 24, 60, 62.  Always rescale (tau 0): every new running
    maximum after the first key moves the reference -- 5 per row.  tau 8: row 0 moves at
    9 (gap 9) and 30 (gap 21): 2; row 1 at 10, 24 (gap 14 over 10; 18 is only 8 above 10:
    delta = -8 keeps the reference) and 60: 3 -- the tie at exactly -8 is a near tie."""
    a = np.array([0.0, 5.0, 9.0, 12.0, 30.0, 31.0])
    q = np.array([[1.0], [2.0]])
    k = a[:, None]
    v = np.eye(6)
    scale = math.log(2.0)
    r0 = model.fa4_forward(q, k, v, scale, block_n=1, threshold=0.0)
    assert list(r0["rescale_rows"]) == [5, 5] and r0["rescales"] == 10
    r8 = model.fa4_forward(q, k, v, scale, block_n=1, threshold=8.0, trace=True)
    assert list(r8["rescale_rows"]) == [2, 3] and r8["rescales"] == 5
    assert list(r8["near_ties"]) == [0, 1]
    # which blocks move, not only how many: the reference after each block, by hand
    # (row 1 keeps 10 at 18, where delta is exactly -8; a strict test would move there
    # and still count 3 moves: 10, 18, 60)
    refs = np.array([st["row_max"] for st in r8["trace"]])
    assert refs[:, 0].tolist() == [0.0, 0.0, 9.0, 9.0, 30.0, 30.0]
    assert refs[:, 1].tolist() == [0.0, 10.0, 10.0, 24.0, 60.0, 60.0]
    # the per-row counts add up to the total on a random causal problem
    rng = np.random.default_rng(9)
    qq, kk, vv = (rng.standard_normal((100, 8)) for _ in range(3))
    kk[rng.choice(100, 3, replace=False)] *= 8.0
    for tau in (0.0, 8.0):
        r = model.fa4_forward(qq, kk, vv, 0.5, causal=True, block_n=16, threshold=tau)
        assert int(r["rescale_rows"].sum()) == r["rescales"]
