"""Fit of the erf-form GELU used by the batched and decode MLP kernels.

GELU(x) = x * Phi(x).  Phi is evaluated as 0.5 + c * P(c^2) with c = x clamped
to [-X, X], X = 3.71875 (119/32, exact in fp32), and P a polynomial of degree
6: the odd part of Phi divided by x is smooth in x^2, so iteratively
reweighted least squares on Chebyshev points of [-X, X] (weights growing where
the |Phi| error peaks, a minimax refinement) balances the error inside the
interval against the clamp's (Phi(X) = 0.99990) at max |Phi error| 5.2e-5 --
as small as a degree-7 fit on [-4, 4], with one operation fewer.  Evaluated in
fp32: one clamp, one multiply, six multiply-adds for P, one multiply-add and one
multiply -- no exponential, no reciprocal (each of those costs four issue slots).

Run to print the coefficients (p0 .. p6, powers of x^2) that
csrc/device_common.hpp carries and the error they reach when evaluated in fp32
(the clamp bound scan: X = 3.70 / 3.71875 / 3.75 / 4.0 give 5.9e-5 / 5.2e-5 /
5.6e-5 / 1.0e-4 at degree 6).
"""
import numpy as np
from scipy.special import ndtr

X, DEG = 3.71875, 6


def fit(X=X, deg=DEG, n=8001, rounds=60):
    xs = np.cos(np.linspace(0, np.pi, n)) * X
    xs = xs[np.abs(xs) > 1e-9]
    target = (ndtr(xs) - 0.5) / xs
    v = xs * xs / (X * X)                       # in [0, 1] for a well-conditioned solve
    A = np.vstack([v ** k for k in range(deg + 1)]).T
    w = np.abs(xs)
    c = np.linalg.lstsq(A * w[:, None], target * w, rcond=None)[0]
    for _ in range(rounds):
        e = np.abs((A @ c - target) * xs)
        w = w * (1 + 2 * e / e.max())
        c = np.linalg.lstsq(A * w[:, None], target * w, rcond=None)[0]
    return (c / (X * X) ** np.arange(deg + 1)).astype(np.float32)


def gelu_fp32(x, p):
    """x * (0.5 + c * P(c^2)), c = clamp(x, -X, X), in fp32 as the kernels evaluate it."""
    x = np.asarray(x, dtype=np.float32)
    c = np.clip(x, np.float32(-X), np.float32(X))
    u = (c * c).astype(np.float32)
    acc = np.float32(p[-1])
    for k in range(len(p) - 2, -1, -1):
        acc = (acc * u + np.float32(p[k])).astype(np.float32)
    return (x * (c * acc + np.float32(0.5))).astype(np.float32)


if __name__ == "__main__":
    p = fit()
    xx = np.linspace(-14, 14, 2800001)
    err = np.abs(gelu_fp32(xx, p).astype(np.float64) - xx * ndtr(xx))
    phi = np.abs(gelu_fp32(xx, p).astype(np.float64) / np.where(xx == 0, 1, xx) - ndtr(xx))[np.abs(xx) > 1e-3]
    print("max |Phi error| %.3e, max |GELU error| %.3e" % (phi.max(), err.max()))
    print("p0..p%d:" % (len(p) - 1), ", ".join("%.8e" % v for v in p))
