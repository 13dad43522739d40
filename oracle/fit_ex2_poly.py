"""Fit of the degree-4 and degree-5 polynomials of the software exp2 (test
infrastructure only; see the package docstring).

"FlashAttention-4's Softmax Tricks: A Degree-3 exp2 on the FMA Pipe, and a
Lagging Max That Saturated FP8", section "The emulated exp2", prints the
degree-3 coefficients (a relative-error minimax fit with p(0) = 1) and the
measured errors of degrees 3, 4 and 5, but not the degree-4 and degree-5
coefficients. They are fitted here the same way:

  1. Remez exchange for  min over c of  max over x in [0, 1] of
     |(1 + c1 x + ... + cn x^n) / 2^x - 1|   (relative error, p(0) = 1);
  2. round c to float32, then lower the measured error of the float32 Horner
     evaluation (one fused multiply-add per step) by moving one coefficient
     at a time by a few float32 steps while the maximum over 2^20 fractions
     in [0, 1) drops.

    python -m oracle.fit_ex2_poly      # prints the coefficients

The results are written out in ex2_emu.c; tests/test_oracle_ex2_poly.py
re-runs this fit and pins those coefficients to the printed error table.
"""
from __future__ import annotations

import math

import numpy as np


def remez_relative(n: int, iters: int = 40):
    """Real coefficients c1..cn of the degree-n relative-error minimax fit
    of 2^x on [0, 1] with constant term 1, and its levelled error."""
    pts = np.array([0.5 * (1.0 - math.cos(math.pi * (i + 1) / (n + 1))) for i in range(n + 1)])
    grid = np.linspace(0.0, 1.0, 200001)
    c, lev = None, None
    for _ in range(iters):
        # 1 + sum c_k x_i^k - 2^x_i = (-1)^i E 2^x_i at the n+1 reference points
        a = np.zeros((n + 1, n + 1))
        b = np.empty(n + 1)
        for i, x in enumerate(pts):
            a[i, :n] = [x ** k for k in range(1, n + 1)]
            a[i, n] = -((-1.0) ** i) * 2.0 ** x
            b[i] = 2.0 ** x - 1.0
        sol = np.linalg.solve(a, b)
        c, lev = sol[:n], abs(sol[n])
        err = (1.0 + sum(c[k - 1] * grid ** k for k in range(1, n + 1))) / 2.0 ** grid - 1.0
        sign = np.sign(err)
        sign[0] = sign[1]
        cuts = [0] + list(np.where(np.diff(sign) != 0)[0] + 1) + [grid.size]
        ext = [lo + int(np.argmax(np.abs(err[lo:hi]))) for lo, hi in zip(cuts[:-1], cuts[1:])]
        if len(ext) != n + 1:
            ext = sorted(sorted(ext, key=lambda j: -abs(err[j]))[:n + 1])
        pts = grid[ext]
    return c, lev


def horner_f32(coef32: np.ndarray, x: np.ndarray) -> np.ndarray:
    """p(x) in float32 Horner form, highest coefficient first, each step one
    correctly rounded fused multiply-add (the float64 product of two float32
    values is exact, the sum is rounded once)."""
    p = np.full(x.shape, coef32[-1], dtype=np.float32)
    for ck in coef32[-2::-1]:
        p = (p.astype(np.float64) * x.astype(np.float64) + np.float64(ck)).astype(np.float32)
    return p


_GRID = np.arange(1 << 20, dtype=np.float64) / (1 << 20)   # exact in float32


def max_rel_error(coef32: np.ndarray) -> float:
    g = _GRID.astype(np.float32)
    return float(np.max(np.abs(horner_f32(coef32, g).astype(np.float64) / np.exp2(_GRID) - 1.0)))


def fit_ex2_poly(n: int) -> np.ndarray:
    """float32 coefficients [1, c1, ..., cn] of the degree-n software exp2."""
    c, _ = remez_relative(n)
    coef = np.array([1.0] + list(c), dtype=np.float32)
    best = max_rel_error(coef)
    improved = True
    while improved:
        improved = False
        for k in range(1, n + 1):
            for steps in (1, -1, 2, -2, 4, -4, 8, -8):
                t = coef.copy()
                t[k] = np.float32(float(t[k]) + steps * float(np.spacing(t[k])))
                e = max_rel_error(t)
                if e < best:
                    best, coef, improved = e, t, True
    return coef


if __name__ == "__main__":
    for deg in (4, 5):
        coef = fit_ex2_poly(deg)
        print(f"degree {deg}: max rel error over the grid {max_rel_error(coef):.4g}")
        for k, v in enumerate(coef):
            print(f"  c{k} = {float(v)!r:<24} ({float(v).hex()})")
