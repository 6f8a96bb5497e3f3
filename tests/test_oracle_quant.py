"""Pins of the oracle's quantization, packing and dequantized product."""

import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import quant, rpbh


def test_threshold_count_equals_bruteforce_argmin():
    for d, bits in ((256, 4), (3072, 2), (3072, 8)):
        c, th, _, _ = cb.lloyd_max_fd(d, bits)
        rng = np.random.default_rng(bits)
        u = rng.standard_normal(200_000) * 1.3 / math.sqrt(d)
        u = np.concatenate([u, c, -1.0 + 0 * c[:1], 1.0 + 0 * c[:1]])
        got = quant.nearest_index(u, th)
        dist = np.abs(u[:, None] - c[None, :])
        want = np.argmin(dist, axis=1)       # first index on ties
        np.testing.assert_array_equal(got, want)


def test_tie_takes_lower_centroid():
    c = np.array([-3.0, -1.0, 1.0, 3.0])
    th = 0.5 * (c[:-1] + c[1:])
    np.testing.assert_array_equal(quant.nearest_index(np.array([-2.0, 0.0, 2.0, 2.0000001]), th), [0, 1, 2, 3])


def test_pack_layout_by_hand():
    idx4 = np.array([[1, 2, 15, 0, 7, 8]])
    np.testing.assert_array_equal(quant.pack(idx4, 4), [[0x21, 0x0F, 0x87]])
    idx2 = np.array([[1, 2, 3, 0, 3, 3, 3, 3]])
    np.testing.assert_array_equal(quant.pack(idx2, 2), [[0b00111001, 0xFF]])
    idx8 = np.array([[0, 255, 17]])
    np.testing.assert_array_equal(quant.pack(idx8, 8), [[0, 255, 17]])
    # 3 bits: sum_k idx_k << 3k = 0x1F58D1, little-endian bytes
    idx3 = np.array([[1, 2, 3, 4, 5, 6, 7, 0]])
    np.testing.assert_array_equal(quant.pack(idx3, 3), [[0xD1, 0x58, 0x1F]])
    # 6 bits: 1 + 63 << 6 + 32 << 12 + 5 << 18 = 0x160FC1
    idx6 = np.array([[1, 63, 32, 5]])
    np.testing.assert_array_equal(quant.pack(idx6, 6), [[0xC1, 0x0F, 0x16]])


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    idx = rng.integers(0, 1 << bits, size=(7, 64))
    p = quant.pack(idx, bits)
    assert p.shape == (7, 64 * bits // 8) and p.dtype == np.uint8
    np.testing.assert_array_equal(quant.unpack(p, bits, 64), idx)


def test_activation_quantization_small_bruteforce():
    # dense R, explicit normalisation and argmin, element by element
    d, h = 64, 16
    perm, sign = rpbh.build_rpbh(d, h, 5)
    R = rpbh.dense_rotation(perm, sign, h)
    c, th, _, _ = cb.lloyd_max_fd(d, 4)
    X = np.random.default_rng(0).standard_normal((6, d)) * 3
    idx, s, x_rot, u = quant.quantize_activations(X, perm, sign, h, th)
    for t in range(6):
        xr = R @ X[t]
        st = math.sqrt(sum(v * v for v in xr))
        assert abs(s[t] - st) < 1e-12 * st
        assert abs(st - np.linalg.norm(X[t])) < 1e-12 * st       # orthogonal
        for k in range(d):
            ut = xr[k] / (st + quant.EPS)
            assert idx[t, k] == int(np.argmin(np.abs(ut - c)))


def test_zero_row_maps_to_center():
    d, h = 64, 64
    perm, sign = rpbh.build_rpbh(d, h, 0)
    _, th, _, _ = cb.lloyd_max_fd(d, 4)
    idx, s, _, _ = quant.quantize_activations(np.zeros((1, d)), perm, sign, h, th)
    assert s[0] == 0.0
    assert np.all(idx == 7)    # #{theta < 0} = L/2 - 1


def test_weight_rows_unit_after_normalisation():
    d, h = 256, 64
    perm, sign = rpbh.build_rpbh(d, h, 0)
    _, th, _, _ = cb.lloyd_max_fd(d, 4)
    W = np.random.default_rng(3).standard_normal((20, d))
    idx, n, w_rot, u = quant.quantize_weights(W, perm, sign, h, th)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(n, np.linalg.norm(W, axis=1), rtol=1e-12)


@pytest.mark.parametrize("bw,ba", [(4, 4), (2, 4), (4, 8), (8, 8)])
def test_product_error_matches_lloyd_max_distortion(bw, ba):
    """The dequantized product approximates W x with the relative error the
    codebooks' distortion predicts: E||y - Wx||^2 / ||Wx||^2 ~ d (D_w + D_a)
    for structureless inputs.  A transposed operand, a wrong index or sign,
    or a missing scale fails this by orders of magnitude."""
    d, h, T, N = 1024, 256, 256, 384
    perm, sign = rpbh.build_rpbh(d, h, 0)
    c_w, th_w, D_w, _ = cb.lloyd_max_fd(d, bw)
    c_a, th_a, D_a, _ = cb.lloyd_max_fd(d, ba)
    rng = np.random.default_rng(bw * 10 + ba)
    X = rng.standard_normal((T, d)) * rng.lognormal(0, 0.5, (T, 1))
    W = rng.standard_normal((N, d)) / math.sqrt(d)
    ia, s, _, _ = quant.quantize_activations(X, perm, sign, h, th_a)
    iw, n, _, _ = quant.quantize_weights(W, perm, sign, h, th_w)
    y = quant.dequantized_product(ia, s, iw, n, c_a, c_w)
    ref = X @ W.T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    pred = math.sqrt(d * D_w + d * D_a)
    assert 0.8 * pred < rel < 1.2 * pred, (rel, pred)


def test_product_bias_and_gelu():
    ia = np.array([[0, 1], [1, 1]])
    iw = np.array([[1, 0]])
    c = np.array([-1.0, 2.0])
    y = quant.dequantized_product(ia, [1.0, 0.5], iw, [2.0], c, c, bias=[0.25])
    # row 0: 1*2*(c0*c1 + c1*c0) = 2*(-2-2) = -8 ; row 1: 0.5*2*(2*2 + 2*-1) = 2
    np.testing.assert_allclose(y[:, 0], [-8 + 0.25, 2 + 0.25])
    g = quant.gelu_erf(np.array([0.0, 1.0, -1.0, 10.0]))
    # GELU(y) = y Phi(y); Phi(1) = 0.8413447460685429 (normal table)
    np.testing.assert_allclose(g, [0.0, 0.8413447460685429, -0.15865525393145707, 10.0], rtol=1e-15, atol=1e-300)


def test_boundary_distance():
    th = np.array([-1.0, 0.0, 2.0])
    dist, near = quant.boundary_distance(np.array([-0.9, 0.1, 1.5, 5.0]), th)
    np.testing.assert_allclose(dist, [0.1, 0.1, 0.5, 3.0])
    np.testing.assert_allclose(near, [-1.0, 0.0, 2.0, 2.0])
