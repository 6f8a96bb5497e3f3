"""Pins of the oracle's marginal f_d and Lloyd-Max solver against closed
forms, quadrature, the uniform special case and the Gaussian Lloyd-Max
table (Max 1960)."""

import json
import math
import os

import mpmath
import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb


def _quad(f, a, b, d):
    # split at the bulk so quad resolves the peak of width 1/sqrt(d)
    s = 1.0 / math.sqrt(d)
    pts = sorted({max(a, min(b, p)) for p in (-12 * s, -8 * s, -4 * s, -2 * s, -s, 0.0, s, 2 * s, 4 * s, 8 * s, 12 * s)} | {a, b})
    tot = 0.0
    for lo, hi in zip(pts[:-1], pts[1:]):
        if hi > lo:
            tot += integrate.quad(f, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
    return tot


@pytest.mark.parametrize("d", [3, 4, 17, 256, 3072, 12288])
def test_fd_normalised_and_variance(d):
    m = cb.SphereMarginal(d)
    assert abs(float(m.mass(-1.0, 1.0)) - 1.0) < 1e-13
    assert abs(_quad(lambda t: float(m.pdf(t)), -1, 1, d) - 1.0) < 1e-12
    # E[t^2] = 1/d exactly for a coordinate of a uniform unit vector
    assert abs(_quad(lambda t: t * t * float(m.pdf(t)), -1, 1, d) * d - 1.0) < 1e-11


@pytest.mark.parametrize("d", [3, 5, 256, 3072])
def test_fd_mass_and_moment_match_quadrature(d):
    m = cb.SphereMarginal(d)
    rng = np.random.default_rng(d)
    s = 1.0 / math.sqrt(d)
    for _ in range(6):
        a, b = np.sort(rng.uniform(-4 * s, 4 * s, 2).clip(-1, 1))
        assert abs(float(m.mass(a, b)) - _quad(lambda t: float(m.pdf(t)), a, b, d)) < 1e-13
        mom = _quad(lambda t: t * float(m.pdf(t)), a, b, d)
        assert abs(float(m.moment1(a, b)) - mom) < 1e-13 * max(1.0, d ** 0.5)


def test_d3_is_uniform_and_its_codebook():
    m = cb.SphereMarginal(3)
    t = np.linspace(-0.99, 0.99, 11)
    np.testing.assert_allclose(m.pdf(t), 0.5, rtol=0, atol=1e-15)
    # Lloyd-Max for the uniform density on [-1, 1] is the uniform quantizer
    c, th, mse, res = cb.lloyd_max_fd(3, 2)
    np.testing.assert_allclose(c, [-0.75, -0.25, 0.25, 0.75], atol=1e-12)
    np.testing.assert_allclose(th, [-0.5, 0.0, 0.5], atol=1e-12)
    assert abs(mse - (0.5 ** 2) / 12) < 1e-13   # step^2 / 12


@pytest.mark.parametrize("d", [4, 256, 3072, 12288])
def test_one_bit_closed_form(d):
    # L = 2: centroids are -/+ E|t| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, th, mse, _ = cb.lloyd_max_fd(d, 1)
    mpmath.mp.dps = 40
    e_abs = float(mpmath.gamma(mpmath.mpf(d) / 2) / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(mpmath.mpf(d + 1) / 2)))
    np.testing.assert_allclose(c, [-e_abs, e_abs], rtol=1e-12)
    assert th[0] == 0.0
    assert abs(mse - (1.0 / d - e_abs ** 2)) < 1e-14


@pytest.mark.parametrize("d,bits", [(256, 4), (3072, 2), (3072, 4), (3072, 8), (5120, 4), (12288, 2), (12288, 8)])
def test_lloyd_max_fixed_point(d, bits):
    dens = cb.SphereMarginal(d)
    c, th, mse, res = cb.lloyd_max_fd(d, bits)
    L = 1 << bits
    assert c.shape == (L,) and th.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(th, 0.5 * (c[:-1] + c[1:]))
    np.testing.assert_allclose(c, -c[::-1], atol=0)
    m, P = cb.conditional_means(c, dens)
    assert np.max(np.abs(c - m)) / np.max(np.abs(c)) <= 1e-10
    assert abs(np.sum(P) - 1.0) < 1e-13
    # at the fixed point sum_j P_j c_j^2 = E[t^2] - MSE
    assert abs(np.sum(P * c * c) - (1.0 / d - mse)) < 1e-10 / d
    assert 0 < mse < 1.0 / d


def _tol(s):
    # one unit of the last printed digit: Max's 1960 hand/early-computer
    # values are off by up to about one unit there (e.g. 0.5006 vs 0.50055)
    dec = len(s.split(".")[1]) if "." in s else 0
    return 10 ** (-dec) + 1e-12


@pytest.mark.parametrize("L", ["2", "4", "8", "16"])
def test_gaussian_lloyd_max_matches_max_1960(golden_dir, L):
    tab = json.load(open(os.path.join(golden_dir, "max1960_gaussian.json")))["tables"][L]
    c, th, mse, res = cb.lloyd_max_gauss(int(L))
    n = int(L)
    for got, want in zip(c[n // 2:], tab["levels"]):
        assert abs(got - float(want)) <= _tol(want), (got, want)
    for got, want in zip(th[n // 2 - 1:], tab.get("thresholds", [])):
        assert abs(got - float(want)) <= _tol(want), (got, want)
    if "mse" in tab:
        assert abs(mse - float(tab["mse"])) <= _tol(tab["mse"])
    if n == 2:
        assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-14
        assert abs(mse - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("bits", [2, 4])
def test_fd_codebook_approaches_scaled_gaussian(bits):
    # "for d > 64 the marginal is essentially N(0, 1/d)": sqrt(d) c_d -> g,
    # with an error that falls like 1/d
    L = 1 << bits
    g, _, gmse, _ = cb.lloyd_max_gauss(L)
    errs = {}
    for d in (256, 1024, 4096):
        c, _, mse, _ = cb.lloyd_max_fd(d, bits)
        errs[d] = np.max(np.abs(math.sqrt(d) * c - g))
        assert errs[d] < 5.0 * L / d
        assert abs(d * mse - gmse) < 20.0 / d
    r1 = errs[256] * 256 / (errs[1024] * 1024)
    r2 = errs[1024] * 1024 / (errs[4096] * 4096)
    assert 0.8 < r1 < 1.25 and 0.8 < r2 < 1.25


def test_fd_256_level_codebook_approaches_scaled_gaussian():
    g, _, _, _ = cb.lloyd_max_gauss(256)
    e = {}
    for d in (3072, 12288):
        c, _, _, res = cb.lloyd_max_fd(d, 8)
        assert res < 1e-10
        e[d] = np.max(np.abs(math.sqrt(d) * c - g)) * d
    assert 0.9 < e[3072] / e[12288] < 1.1
