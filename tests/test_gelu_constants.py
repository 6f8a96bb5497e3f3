"""The GELU epilogue's constants (qlinear.hip, gelu_erf), checked on the CPU.

The kernel evaluates GELU(v) = v Phi(v) through the Mills ratio
R(z) = (1 - Phi(z)) / phi(z) of the standard normal, approximated by a
rational function of degree 4 / 5.  This test reads the coefficients from the
kernel source, checks the rational function against sqrt(pi / 2)
erfcx(z / sqrt 2) on [0, 13], and replays the kernel's fp32 formula step by
step (numpy float32 rounding after every operation; exp2 and the reciprocal
correctly rounded) against fp64 GELU, so that a mistyped coefficient or a
dropped correction term fails here before any GPU run.  The GPU test of the
epilogue itself is test_gelu_epilogue_matches_fp64_gelu_of_the_gpu_output."""

import os
import re

import numpy as np
import pytest

special = pytest.importorskip("scipy.special")

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "free_bit_quantization_amd", "csrc", "qlinear.hip")


def _body():
    s = open(SRC).read()
    i = s.index("__device__ __forceinline__ float gelu_erf(float v) {")
    return s[i:s.index("\n}", i)]


def _horner(name, body):
    # const float p = fmaf(fmaf(...(c_n, z, c_{n-1}), z, ...), z, c_0);
    m = re.search(r"const float " + name + r" = (.*?);", body, re.S)
    nums = [float(x) for x in re.findall(r"([0-9]+\.[0-9]+(?:e-?[0-9]+)?)f", m.group(1))]
    return nums   # highest degree first


def test_rational_mills_ratio_on_0_13():
    body = _body()
    p, q = _horner("p", body), _horner("q", body)
    assert len(p) == 5 and len(q) == 6
    z = np.linspace(0.0, 13.0, 200001)
    approx = np.polyval(p, z) / np.polyval(q, z)
    exact = np.sqrt(np.pi / 2) * special.erfcx(z / np.sqrt(2))
    assert np.max(np.abs(approx / exact - 1)) < 1e-7


def test_fp32_replay_of_the_kernel_formula():
    body = _body()
    p, q = _horner("p", body), _horner("q", body)
    consts = dict(re.findall(r"(kLog2eHi|kLog2eLo|kLn2|kInvSqrt2Pi) = ([0-9.e-]+)f", body))
    f32 = np.float32

    def r(x):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)

    def fma(a, b, c):   # one rounding (the float64 product of two float32 is exact)
        return r(np.asarray(a, dtype=np.float64) * b + c)

    Lh, Ll = float(f32(consts["kLog2eHi"])), float(f32(consts["kLog2eLo"]))
    ln2, c0 = float(f32(consts["kLn2"])), float(f32(consts["kInvSqrt2Pi"]))
    v = r(np.linspace(-9.0, 9.0, 400001))
    z = np.abs(v)
    pp = np.full_like(z, r(p[0]))
    for c in p[1:]:
        pp = fma(pp, z, r(c))
    qq = np.full_like(z, r(q[0]))
    for c in q[1:]:
        qq = fma(qq, z, r(c))
    rr = r(pp * r(1.0 / qq))
    vv = r(v * v)
    vv_lo = fma(v, v, -vv)
    h = r(0.5 * vv)
    t = r(h * Lh)
    t_lo = fma(h, Ll, fma(h, Lh, -t))
    ex = r(np.exp2(-t))
    ex = fma(fma(-0.5, vv_lo, r(-t_lo * ln2)), ex, ex)
    lower = r(r(ex * c0) * rr)
    g = r(v * np.where(v <= 0, lower, r(1.0 - lower)))
    exact = v * 0.5 * special.erfc(-v / np.sqrt(2))
    ok = exact != 0
    assert np.max(np.abs(g[ok] / exact[ok] - 1)) < 8e-7
