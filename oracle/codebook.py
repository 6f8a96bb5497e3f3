"""The fixed marginal f_d and its Lloyd-Max codebook, fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Method ("OrbitQuant: data-agnostic quantization for image and video",
rcap.io summary, "core trick" paragraph and the offline pseudo-code line
``codebook[d, b] = lloyd_max(f_d, b)``): every coordinate of a randomly
rotated unit vector in R^d follows one marginal that depends only on d;
one optimal scalar quantizer (the standard Lloyd-Max construction, 2^b
centroids) is built for it offline.  The aiweekly.co news item adds that
one codebook serves every layer of a given input dimension.

The exact marginal of one coordinate of a uniform point on the sphere
S^{d-1} (a textbook fact; the page only says it approaches N(0, 1/d) for
d > 64):

    f_d(t) = C_d (1 - t^2)^((d-3)/2)  on [-1, 1],
    C_d    = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).

Equivalently (1 + t)/2 ~ Beta((d-1)/2, (d-1)/2), so the CDF is a
regularised incomplete beta function (scipy's ``betainc`` is the step).
The partial first moment has a closed form,

    int_a^b t f_d(t) dt = C_d / (d-1) * [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)].

Lloyd-Max (Lloyd 1957 / Max 1960): L = 2^b centroids c_0 < ... < c_{L-1}
and thresholds theta_j = (c_j + c_{j+1})/2 are optimal when each centroid
is the conditional mean of its cell, c_j = E[t | theta_{j-1} < t <= theta_j]
(theta_{-1}, theta_{L-1} = the ends of the support).  The oracle iterates
those two conditions and then solves the fixed point by Newton's method
on G(c) = c - m(c), whose Jacobian is tridiagonal (readings: start at
quantiles of N(0, 3/d), the f^(1/3) compander rule; symmetry of the
codebook enforced; stop on a residual of ~1e-14 * max|c|).  f_d is
log-concave for d >= 3, so the fixed point is unique and the start does
not change it.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np
from scipy import special


# --------------------------------------------------------------------------
# Densities: each exposes support, pdf, mass(a, b), moment1(a, b), second
# moment E[t^2], and an initial spread for the compander start.
# --------------------------------------------------------------------------


class SphereMarginal:
    """f_d, the marginal of one coordinate of a uniform unit vector in R^d."""

    def __init__(self, d: int):
        if d < 3:
            raise ValueError("f_d needs d >= 3")
        self.d = d
        self.a = (d - 1) / 2.0
        # C_d from 40-digit Gamma values: the difference of two fp64 gammaln
        # values near 5e4 (d = 12288) would lose ~4e-12 relative accuracy
        mpmath.mp.dps = 40
        self.log_c = float(mpmath.log(mpmath.gamma(mpmath.mpf(d) / 2)
                                      / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(mpmath.mpf(d - 1) / 2))))
        self.lo, self.hi = -1.0, 1.0
        self.second_moment = 1.0 / d
        self.sigma = 1.0 / math.sqrt(d)

    def pdf(self, t):
        t = np.asarray(t, dtype=np.float64)
        inside = np.abs(t) < 1.0
        tt = np.where(inside, t, 0.0)
        val = np.exp(self.log_c + 0.5 * (self.d - 3) * np.log1p(-tt * tt))
        edge = np.exp(self.log_c) if self.d == 3 else 0.0   # value at |t| == 1
        return np.where(inside, val, np.where(np.abs(t) == 1.0, edge, 0.0))

    def _lower(self, t):
        # P(T <= t), accurate in the lower tail
        return special.betainc(self.a, self.a, (1.0 + t) / 2.0)

    def _upper(self, t):
        # P(T > t), accurate in the upper tail (symmetry of f_d)
        return special.betainc(self.a, self.a, (1.0 - t) / 2.0)

    def mass(self, a, b):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        return np.where(b <= 0.0, self._lower(b) - self._lower(a),
                        np.where(a >= 0.0, self._upper(a) - self._upper(b),
                                 1.0 - self._lower(a) - self._upper(b)))

    def moment1(self, a, b):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        e = (self.d - 1) / 2.0

        def g(t):
            t = np.clip(t, -1.0, 1.0)
            with np.errstate(divide="ignore"):
                return np.exp(e * np.log1p(-t * t))

        return np.exp(self.log_c) / (self.d - 1) * (g(a) - g(b))


class Gaussian:
    """N(0, 1): the limit the page names for d > 64 (after scaling by sqrt(d))."""

    def __init__(self):
        self.lo, self.hi = -np.inf, np.inf
        self.second_moment = 1.0
        self.sigma = 1.0

    def pdf(self, t):
        t = np.asarray(t, dtype=np.float64)
        return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)

    def mass(self, a, b):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        return np.where(b <= 0.0, special.ndtr(b) - special.ndtr(a), special.ndtr(-a) - special.ndtr(-b))

    def moment1(self, a, b):
        return self.pdf(a) - self.pdf(b)


# --------------------------------------------------------------------------
# Lloyd-Max
# --------------------------------------------------------------------------


def _cells(c, dens):
    theta = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([dens.lo], theta))
    hi = np.concatenate((theta, [dens.hi]))
    return theta, lo, hi


def conditional_means(c, dens):
    """m_j = E[t | cell j] for the midpoint cells of centroids c, and P_j."""
    _, lo, hi = _cells(c, dens)
    P = dens.mass(lo, hi)
    M = dens.moment1(lo, hi)
    return M / P, P


def lloyd_max(dens, L: int, lloyd_steps: int = 50, newton_steps: int = 200, tol: float = 1e-14):
    """Solve the Lloyd-Max conditions for ``dens`` with L levels.

    Returns (centroids[L], thresholds[L-1], mse, residual) where residual is
    max_j |c_j - E[t | cell_j]| / max|c| at the returned point.
    """
    if L < 2:
        raise ValueError("L >= 2")
    # compander start: quantiles of N(0, 3 sigma^2) at (j + 1/2)/L
    p = (np.arange(L) + 0.5) / L
    c = math.sqrt(3.0) * dens.sigma * special.ndtri(p)
    if np.isfinite(dens.hi) and np.max(np.abs(c)) > 0.95 * dens.hi:
        c *= 0.95 * dens.hi / np.max(np.abs(c))    # keep the start inside a bounded support
    c = 0.5 * (c - c[::-1])

    for _ in range(lloyd_steps):
        m, _ = conditional_means(c, dens)
        c = 0.5 * (m - m[::-1])

    def resid(cv):
        m, P = conditional_means(cv, dens)
        return cv - m, m, P

    G, m, P = resid(c)
    best = np.max(np.abs(G))
    for _ in range(newton_steps):
        if best <= tol * np.max(np.abs(c)):
            break
        theta, lo, hi = _cells(c, dens)
        # d m_j / d theta_{j-1} and d m_j / d theta_j (zero at fixed ends)
        f_lo = np.where(np.isfinite(lo), dens.pdf(np.where(np.isfinite(lo), lo, 0.0)), 0.0)
        f_hi = np.where(np.isfinite(hi), dens.pdf(np.where(np.isfinite(hi), hi, 0.0)), 0.0)
        f_lo[0] = 0.0
        f_hi[-1] = 0.0
        lo_f = np.where(np.isfinite(lo), lo, 0.0)
        hi_f = np.where(np.isfinite(hi), hi, 0.0)
        a = f_lo * (m - lo_f) / P
        b = f_hi * (hi_f - m) / P
        # theta_j = (c_j + c_{j+1}) / 2  ->  dm/dc is tridiagonal
        J = np.eye(L)
        idx = np.arange(L)
        J[idx, idx] -= 0.5 * (a + b)
        J[idx[1:], idx[1:] - 1] -= 0.5 * a[1:]
        J[idx[:-1], idx[:-1] + 1] -= 0.5 * b[:-1]
        step = np.linalg.solve(J, -G)
        lam = 1.0
        improved = False
        while lam > 1e-4:
            cn = c + lam * step
            cn = 0.5 * (cn - cn[::-1])
            if np.all(np.diff(cn) > 0):
                Gn, mn, Pn = resid(cn)
                rn = np.max(np.abs(Gn))
                if rn < best:
                    c, G, m, P, best = cn, Gn, mn, Pn, rn
                    improved = True
                    break
            lam *= 0.5
        if not improved:
            break

    theta = 0.5 * (c[:-1] + c[1:])
    _, lo, hi = _cells(c, dens)
    Pm = dens.mass(lo, hi)
    Mm = dens.moment1(lo, hi)
    mse = dens.second_moment - 2.0 * np.sum(c * Mm) + np.sum(c * c * Pm)
    return c, theta, float(mse), float(best / np.max(np.abs(c)))


def lloyd_max_fd(d: int, bits: int):
    """Codebook for f_d with 2^bits levels: (centroids, thresholds, mse, residual)."""
    return lloyd_max(SphereMarginal(d), 1 << bits)


def lloyd_max_gauss(L: int):
    """Codebook for N(0, 1) with L levels: (centroids, thresholds, mse, residual)."""
    return lloyd_max(Gaussian(), L)
