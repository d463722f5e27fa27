"""Plant plausible mistakes in copies of the blockwise model (oracle/model.py)
and check that the model's own pins -- the worked example's round states, FA4
exercise 1, the threshold tie, equality with the three-pass oracle, the rescale
counts worked by hand -- catch every one of them.  Runs on the CPU."""
import itertools
import os
import types

import pytest

from oracle import model as _model
from tests import test_model as pins


def _read(path):
    with open(path) as f:
        return f.read()


SRC = _model.__file__

MUTANTS = {
    # the rescale decision: keep the reference while delta >= -tau
    "tie_strict": ("keep = (candidate == -np.inf) | (delta >= -threshold)",
                   "keep = (candidate == -np.inf) | (delta > -threshold)"),
    "row_tie_strict": ("if candidate == -math.inf or delta >= -threshold:",
                       "if candidate == -math.inf or delta > -threshold:"),
    "reference_swapped": ("new_ref = np.where(keep, row_max, candidate)",
                          "new_ref = np.where(keep, candidate, row_max)"),
    # alpha = exp2(delta) rescales the running state
    "alpha_sign": ("np.exp2(np.where(keep, 0.0, delta))", "np.exp2(np.where(keep, 0.0, -delta))"),
    "row_alpha_sign": ("new_ref, acc_scale = candidate, 2.0 ** delta",
                       "new_ref, acc_scale = candidate, 2.0 ** -delta"),
    "sum_not_rescaled": ("row_sum = row_sum * acc_scale + P.sum(axis=1)",
                         "row_sum = row_sum + P.sum(axis=1)"),
    "o_not_rescaled": ("O = block_O if first else O * acc_scale[:, None] + block_O",
                       "O = block_O if first else O + block_O"),
    # mask alignment, LSE units, counters
    "causal_top_left": ("S = np.where(kj > qi + (Nk - Nq), -np.inf, S)",
                        "S = np.where(kj > qi, -np.inf, S)"),
    "lse_in_log2_units": ("lse[nz] = np.log(row_sum[nz]) + row_max[nz] * float(scale)",
                          "lse[nz] = np.log(row_sum[nz]) + row_max[nz] * scale_log2"),
    "rows_count_kept_blocks": ("rescale_rows += ~keep", "rescale_rows += keep"),
    "near_tie_margin_sign": ("np.abs(gap + threshold) < tie_eps", "np.abs(gap - threshold) < tie_eps"),
}

_MATCH_PARAMS = list(itertools.product([False, True], [0.0, 8.0], [False, True],
                                       [(1, 7, 7), (3, 9, 13), (16, 40, 33), (4, 10, 6)]))


def _checks():
    yield pins.test_worked_example_rounds_always_rescale
    yield pins.test_worked_example_rounds_conditional
    yield pins.test_exercise1_keep_reference
    yield pins.test_exercise1_switch_reference
    yield pins.test_exercise1_always_rescale_same_ratio
    yield pins.test_threshold_tie_keeps_reference
    for causal, tau, reverse, (bn, nq, nk) in _MATCH_PARAMS:
        yield lambda c=causal, t=tau, r=reverse, b=bn, q=nq, k=nk: \
            pins.test_model_matches_oracle(c, t, r, b, q, k)
    yield pins.test_outlier_keys_force_rescales
    yield pins.test_fully_masked_first_blocks_stay_finite
    yield pins.test_rescale_counts_per_row_by_hand


def _load(text, name):
    mod = types.ModuleType(name)
    mod.__file__ = f"<{name}>"
    exec(compile(text, mod.__file__, "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(pins, "model", _load(_read(SRC), "model_copy"))
    for check in _checks():
        check()


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # mutants may produce inf * 0
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_model_mutant_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    src = _read(SRC)
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    monkeypatch.setattr(pins, "model", _load(src.replace(old, new), f"model_{name}"))
    caught = 0
    for check in _checks():
        try:
            check()
        except Exception:  # an assertion, a NaN comparison or a crash counts as caught
            caught += 1
    assert caught, f"mutant {name} passed every pin"
