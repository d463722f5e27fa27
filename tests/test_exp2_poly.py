"""The split exp2's polynomial (fa_device.h exp2_poly): its coefficients are
the Remez fit that csrc/fit_exp2_poly.py computes, the fit's minimax relative
error is levelled below 7.5e-5, and the kernel's evaluation (fract, Horner in
fp32 with fused multiply-adds, exponent by ldexp, clamp at -200) stays within
that bound of exp2 over the range the kernel feeds it (x <= 15), with -inf and
deep underflow giving exactly 0.  Pinned against numpy's fp64 exp2."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_forward_fa_amd", "csrc")


def _coefficients():
    src = open(os.path.join(CSRC, "fa_device.h")).read()
    return [float(re.search(rf"kExp2C{i} = ([0-9.e+-]+)f;", src).group(1)) for i in range(4)]


def _fit_module():
    spec = importlib.util.spec_from_file_location("fit_exp2_poly", os.path.join(CSRC, "fit_exp2_poly.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _fma32(a, b, c):
    """fp32 fused multiply-add: the exact a*b + c rounded once to fp32."""
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(np.float32)


def kernel_exp2(x):
    """The device function's arithmetic, step by step, in fp32."""
    c0, c1, c2, c3 = (np.float32(c) for c in _coefficients())
    x = np.maximum(np.asarray(x, dtype=np.float32), np.float32(-200.0))
    j = np.floor(x)
    f = (x - j).astype(np.float32)          # v_fract_f32 is exact for |x| < 2^23
    p = _fma32(_fma32(_fma32(c3, f, c2), f, c1), f, c0)
    return np.ldexp(p, j.astype(np.int32)).astype(np.float32)


def test_coefficients_are_the_remez_fit():
    fit = _fit_module()
    coef, emax, lev = fit.remez()
    assert abs(emax - lev) < 1e-9                      # levelled: the minimax solution
    assert emax < 7.5e-5
    np.testing.assert_allclose(_coefficients(), coef, rtol=0, atol=1e-7)


def test_relative_error_bound_on_the_kernel_range():
    x = np.concatenate([np.linspace(-40.0, 15.0, 2_000_003, dtype=np.float64),
                        np.arange(-40, 16, dtype=np.float64)]).astype(np.float32)
    got = kernel_exp2(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(got / ref - 1.0)
    assert rel.max() < 7.5e-5 + 2e-7, rel.max()       # the fit's bound plus fp32 rounding
    # a fit of lower degree would not meet it: the bound is the cubic's
    assert rel.max() > 5e-5


def test_masked_and_underflow_give_zero():
    out = kernel_exp2(np.array([-np.inf, -1e30, -200.0, -150.5], dtype=np.float32))
    assert np.all(out == 0.0)
    # the reference weight (x = 0) rounds to exactly 1 in fp16, as v_exp_f32's does
    assert np.float16(kernel_exp2(np.float32(0.0))) == np.float16(1.0)
