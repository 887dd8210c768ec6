"""Fit of the erf-form GELU used by the batched MLP kernels.

GELU(x) = x * Phi(x).  Phi is written as sigmoid(p(x)) with p an odd polynomial
of degree 9 fitted to the logit of Phi, log Phi(x) - log Phi(-x): the error of
the logit enters Phi scaled by Phi (1 - Phi), so a weighted least-squares start
refined to minimax on |Phi error| over [0, 9] gives max |Phi error| about
1.5e-6 (odd symmetry covers x < 0; beyond 9 both sides saturate).  Evaluating
x * sigmoid(p(x)) costs five multiply-adds, one exp2 and one reciprocal.

Run to print the coefficients (c1, c3, c5, c7, c9) that csrc/device_common.hpp
carries, pre-multiplied by -log2(e), and the error they reach.
"""
import numpy as np
from scipy.optimize import minimize
from scipy.special import log_ndtr, ndtr

LOG2E = 1.4426950408889634


def fit(deg=5, lo=0.0, hi=9.0, n=20001):
    x = np.linspace(lo, hi, n)
    logit = log_ndtr(x) - log_ndtr(-x)
    w = ndtr(x) * ndtr(-x)

    def phi_err(c):
        u = x * x
        p = np.zeros_like(x)
        for k in reversed(range(deg)):
            p = p * u + c[k]
        return 1.0 / (1.0 + np.exp(-p * x)) - ndtr(x)

    A = np.stack([x ** (2 * k + 1) for k in range(deg)], 1)
    c0 = np.linalg.lstsq(A * w[:, None], logit * w, rcond=None)[0]
    res = minimize(lambda c: np.max(np.abs(phi_err(c))), c0, method="Nelder-Mead",
                   options=dict(maxiter=40000, xatol=1e-14, fatol=1e-14))
    return res.x, float(np.max(np.abs(phi_err(res.x))))


if __name__ == "__main__":
    c, err = fit()
    print("max |Phi error| %.3e" % err)
    print("coefficients c1..c9:", ", ".join("%.17g" % v for v in c))
    print("times -log2(e):     ", ", ".join("%.9e" % (-v * LOG2E) for v in c))
