"""Coefficients of the GELU epilogue (qlinear.hip, gelu_erf).

The epilogue computes Phi(-z) = phi(z) R(z), z = |v|, with R the Mills ratio
of the standard normal, R(z) = (1 - Phi(z)) / phi(z) = sqrt(pi / 2)
erfcx(z / sqrt 2).  R is smooth and positive on [0, inf), R(0) = sqrt(pi / 2),
R(z) ~ 1 / z; it is approximated on [0, 13] (beyond, phi(z) underflows fp32)
by a rational function P(z) / Q(z) of degree 4 / 5, fitted here by
iteratively reweighted least squares on the relative error at Chebyshev
nodes against scipy's erfcx.  Run with python3: it prints the coefficients
(Q's constant term is 1; all come out positive, so Horner's rule does not
cancel for z >= 0) and the fit's maximum relative error in double precision
on a fine grid (~5e-9).
"""
import numpy as np
from scipy import special


def mills_ratio(z):
    return special.erfcx(z / np.sqrt(2.0)) * np.sqrt(np.pi / 2.0)


def fit(m=4, n=5, lo=0.0, hi=13.0, iters=40, nodes=6000):
    x = np.cos(np.linspace(0.0, np.pi, nodes)) * 0.5 * (hi - lo) + 0.5 * (hi + lo)
    f = mills_ratio(x)
    w = np.ones(nodes)
    for _ in range(iters):
        A = np.hstack([x[:, None] ** np.arange(m + 1), -(f[:, None]) * x[:, None] ** np.arange(1, n + 1)])
        c, *_ = np.linalg.lstsq(A * (w / f)[:, None], f * (w / f), rcond=None)
        p, q = c[:m + 1], np.concatenate([[1.0], c[m + 1:]])
        err = (np.polyval(p[::-1], x) / np.polyval(q[::-1], x) - f) / f
        w = w * (np.abs(err) / np.abs(err).mean()) ** 0.3
    xs = np.linspace(lo, hi, 400001)
    fs = mills_ratio(xs)
    worst = np.abs((np.polyval(p[::-1], xs) / np.polyval(q[::-1], xs) - fs) / fs).max()
    return p, q, worst


if __name__ == "__main__":
    p, q, worst = fit()
    print("P (z^0 .. z^4):", ", ".join(f"{float(np.float32(v)):.9g}f" for v in p))
    print("Q (z^0 .. z^5):", ", ".join(f"{float(np.float32(v)):.9g}f" for v in q))
    print(f"max relative error of the fit: {worst:.3g}")
