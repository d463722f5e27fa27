"""Fit the cubic of the forward kernel's polynomial exp2 (fa_device.h, exp2_poly).

2^x is computed as 2^j * p(f) with j = floor(x) and f = x - j in [0, 1), the
2^j applied by the exponent field (v_ldexp_f32).  p is the degree-3 polynomial
that minimises the largest relative error max |p(f) / 2^f - 1| on [0, 1]
(minimax), found by the Remez exchange algorithm: solve for the coefficients
and the levelled error E on n + 2 reference points with alternating signs,
move the references to the extrema of the error curve, repeat until the
extrema are level.  The kernel rounds P to fp16 (relative 2^-11 = 4.9e-4)
after this, so a relative error near 1e-4 is ample.

    python fit_exp2_poly.py      # prints the coefficients and the error bound
"""
import numpy as np

DEGREE = 3


def remez(degree: int = DEGREE, iters: int = 50, grid: int = 200001):
    n = degree
    xs = np.linspace(0.0, 1.0, grid)
    target = np.exp2(xs)
    # Chebyshev-like initial references on [0, 1]
    k = np.arange(n + 2)
    ref = 0.5 - 0.5 * np.cos(np.pi * k / (n + 1))
    coef = None
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i  (relative error levelled at +-E)
        A = np.zeros((n + 2, n + 2))
        for i, x in enumerate(ref):
            A[i, :n + 1] = x ** np.arange(n + 1)
            A[i, n + 1] = -((-1) ** i) * np.exp2(x)
        sol = np.linalg.solve(A, np.exp2(ref))
        coef, E = sol[:n + 1], sol[n + 1]
        err = np.polyval(coef[::-1], xs) / target - 1.0
        # new references: the extremum of each run of constant error sign
        sign = np.sign(err)
        sign[sign == 0] = 1
        runs = np.flatnonzero(np.diff(sign)) + 1
        bounds = np.concatenate([[0], runs, [len(xs)]])
        ext = [b0 + int(np.argmax(np.abs(err[b0:b1]))) for b0, b1 in zip(bounds[:-1], bounds[1:])]
        if len(ext) != n + 2:
            break
        new_ref = xs[ext]
        if np.allclose(new_ref, ref, atol=1e-12, rtol=0):
            break
        ref = new_ref
    err = np.polyval(coef[::-1], xs) / target - 1.0
    return coef, float(np.abs(err).max()), float(abs(E))


if __name__ == "__main__":
    c, emax, lev = remez()
    print(f"degree {DEGREE} minimax relative error {emax:.4e} (levelled {lev:.4e})")
    for i, v in enumerate(c):
        print(f"c{i} = {np.float32(v)!r}  ({v:.17g})")
