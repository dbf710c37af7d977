"""Fit of the scaled complementary error function used by the bf16 epilogues.

erfc(z) = t e^{-z^2} S(t),  t = 1 / (1 + p z),  z >= 0,

with S a polynomial of degree n in t on (0, 1] fitted for least maximum
relative error (iteratively reweighted least squares on Chebyshev-spaced t,
erfc(z) e^{z^2} from scipy.special.erfcx), and p chosen by a grid search.  The
same form as the Chebyshev-fitted erfc of Press et al., Numerical Recipes
(2nd ed., section 6.2), which fits log S instead, to degree 9.  Prints the
coefficients of S / 2 (the epilogues need Phi(-|x|) = erfc(|x| / sqrt 2) / 2)
lowest order first, and the fit's maximum relative error.

Usage: python fit_erfc.py [degree]   (the library uses degree 6)
"""
import sys
import numpy as np
from scipy.special import erfcx


def fit(p, n, nodes=40000, iters=60):
    t = 0.5 * (1.0 - np.cos(np.linspace(0.0, np.pi, nodes)))
    t = t[t > 1e-7]
    z = (1.0 / t - 1.0) / p
    S = erfcx(z) / t
    V = np.vander(t, n + 1, increasing=True)
    w = 1.0 / S
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * w[:, None], S * w, rcond=None)
        err = V @ c / S - 1.0
        w = w * (1.0 + 4.0 * np.abs(err) / np.abs(err).max())
    return float(np.abs(err).max()), c


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 6
    grid = np.round(np.arange(0.30, 0.60001, 0.005), 3)
    err, c, p = min(((*fit(p, n), p) for p in grid), key=lambda r: r[0])
    print(f"degree {n}: p = {p:.3f}, max relative error of S {err:.3e}")
    print("S/2 coefficients, lowest order first:")
    for k, v in enumerate(0.5 * c):
        print(f"  c{k} = {float(np.float32(v)):.9g}")


if __name__ == "__main__":
    main()
