"""Minimax polynomial for 2^f on [0, 1), relative error, by the Remez exchange.

The MHA v4 page ("Motivation") lists exponential approximation/emulation
among its kernel levers, and the FA4 autotuning page names an exp2 emulation
policy: part of a softmax's exponentials computed with FMAs instead of the
transcendental unit.  Evaluated as 2^t = 2^n * p(f) with n = floor(t) and
f = t - n, this needs a polynomial p close to 2^f on [0, 1).  This script
computes it from the mathematics alone -- no published coefficient set is
used: the Remez exchange on the relative error e(f) = p(f) / 2^f - 1 over
degree-d polynomials, in FP64, then the FP32 rounding of the coefficients and
the maximum relative error of their FP32 Horner evaluation on a dense grid.

    python exp2_remez.py [degree ...]      (default: 3 4 5)

prints, per degree, the FP32 coefficients c0..cd (p(f) = c0 + c1 f + ...)
and the measured error.  Used to size the attention kernel's exp2
emulation experiment (the kernel keeps v_exp_f32; see the measurement
recorded with the kernel)."""
import sys

import numpy as np


def remez(deg: int, iters: int = 60):
    """Coefficients (FP64) minimising max |p(f) / 2^f - 1| on [0, 1]."""
    n = deg + 2
    # Chebyshev extrema as the first reference
    x = 0.5 - 0.5 * np.cos(np.pi * np.arange(n) / (n - 1))
    grid = np.linspace(0.0, 1.0, 200001)
    coef = None
    for _ in range(iters):
        # solve p(x_i) - 2^x_i = (-1)^i E 2^x_i  (relative equioscillation)
        A = np.zeros((n, n))
        for i in range(n):
            A[i, :deg + 1] = x[i] ** np.arange(deg + 1)
            A[i, deg + 1] = -((-1) ** i) * 2.0 ** x[i]
        sol = np.linalg.solve(A, 2.0 ** x)
        coef = sol[:deg + 1]
        err = np.polyval(coef[::-1], grid) / 2.0 ** grid - 1.0
        # new reference: the extrema of err between sign changes
        idx = [0]
        for j in range(1, grid.size - 1):
            if (err[j] - err[j - 1]) * (err[j + 1] - err[j]) <= 0:
                idx.append(j)
        idx.append(grid.size - 1)
        idx = np.array(sorted(set(idx)))
        # keep n alternating extrema of largest magnitude
        cand = [(grid[j], err[j]) for j in idx]
        merged = []
        for xv, ev in cand:
            if merged and np.sign(merged[-1][1]) == np.sign(ev):
                if abs(ev) > abs(merged[-1][1]):
                    merged[-1] = (xv, ev)
            else:
                merged.append((xv, ev))
        while len(merged) > n:
            # drop the smaller end
            if abs(merged[0][1]) < abs(merged[-1][1]):
                merged.pop(0)
            else:
                merged.pop()
        if len(merged) < n:
            break
        x = np.array([m[0] for m in merged])
    return coef


def fp32_error(coef32: np.ndarray) -> float:
    f = np.linspace(0.0, 1.0, 1 << 20, endpoint=False).astype(np.float32)
    p = np.full(f.shape, coef32[-1], np.float32)
    for c in coef32[-2::-1]:
        p = (p * f + c).astype(np.float32)   # FMA-free Horner: an upper bound of the FMA form's error
    exact = np.exp2(f.astype(np.float64))
    return float(np.max(np.abs(p.astype(np.float64) / exact - 1.0)))


def main(argv):
    degs = [int(a) for a in argv] or [3, 4, 5]
    for d in degs:
        c = remez(d)
        c32 = c.astype(np.float32)
        print(f"degree {d}: max relative error {fp32_error(c32):.3e} (2^{np.log2(fp32_error(c32)):.1f})")
        print("  " + ", ".join(f"{float(v):.9e}f" for v in c32))


if __name__ == "__main__":
    main(sys.argv[1:])
