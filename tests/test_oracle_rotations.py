"""Rotation variants (rcap.io summary: the RPBH paragraph, whose reference
point is a dense random rotation, and the ablation paragraph, which removes
RPBH's leading permutation -- "Block-RHT").  CPU only.

Pins:
* Block-RHT tables: identity permutation; signs = top bits of the published
  splitmix64 vector for seed 1234567 (tests/golden/splitmix64.json);
* the dense Haar rotation is orthogonal and, because the coordinates of a
  uniformly rotated unit vector follow f_d exactly, its relative
  quantization error equals sqrt(d * D) with D the Lloyd-Max distortion of
  f_d per coordinate (law of large numbers over T*d coordinates);
* the mechanism the ablation paragraph states: with outlier channels
  concentrated in one Hadamard block, Block-RHT quantizes much worse than
  RPBH, and with no outliers the three rotations agree.
"""

import json
import os

import numpy as np
import pytest

from oracle import codebook, quant, rpbh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")


def test_block_rht_tables_from_published_stream():
    vec = next(v for v in json.load(open(GOLDEN))["vectors"] if v["seed"] == 1234567)
    outs = [int(o) for o in vec["outputs"]]
    d, h = 8, 2
    perm, sign = rpbh.build_block_rht(d, h, 1234567)
    assert np.array_equal(perm, np.arange(d))
    expect = [-1 if (o >> 63) else 1 for o in outs]
    assert list(sign[:len(expect)]) == expect


def test_block_rht_is_rpbh_without_permutation():
    # same Hadamard blocks and sign rule: the dense matrix is B D with P = I
    d, h = 64, 16
    perm, sign = rpbh.build_block_rht(d, h, 7)
    R = rpbh.dense_rotation(perm, sign, h)
    B = np.kron(np.eye(d // h), rpbh.sylvester(h) / np.sqrt(h))
    assert np.max(np.abs(R - B @ np.diag(sign.astype(np.float64)))) == 0.0
    assert np.max(np.abs(R @ R.T - np.eye(d))) < 1e-15


def test_haar_rotation_orthogonal_and_seeded():
    Q = rpbh.haar_rotation(128, 3)
    assert np.max(np.abs(Q @ Q.T - np.eye(128))) < 1e-12
    assert np.array_equal(Q, rpbh.haar_rotation(128, 3))
    assert not np.array_equal(Q, rpbh.haar_rotation(128, 4))


def _errors(x, d, h, bits, seed=0):
    c, th, mse, _ = codebook.lloyd_max_fd(d, bits)
    out = {}
    for name, (perm, sign) in (("rpbh", rpbh.build_rpbh(d, h, seed)), ("block_rht", rpbh.build_block_rht(d, h, seed))):
        idx, s, x_rot, _ = quant.quantize_activations(x, perm, sign, h, th)
        out[name] = quant.relative_error(x_rot, idx, s, c)
    x_rot = x @ rpbh.haar_rotation(d, seed).T
    idx, s = quant.quantize_rotated(x_rot, th)
    out["dense"] = quant.relative_error(x_rot, idx, s, c)
    return out, float(np.sqrt(d * mse))


@pytest.mark.parametrize("bits", [2, 4])
def test_dense_rotation_error_is_the_codebook_distortion(bits):
    d, h = 512, 64
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, d)) * np.exp(0.5 * rng.standard_normal((256, 1)))
    x[:, 5:9] *= 40.0   # any input: a Haar rotation makes the marginal exact
    errs, theory = _errors(x, d, h, bits)
    assert abs(errs["dense"] / theory - 1.0) < 0.02, (errs, theory)


def test_permutation_spreads_concentrated_outliers():
    d, h, bits = 1024, 64, 4
    rng = np.random.default_rng(0)
    x = rng.standard_normal((256, d))
    x[:, 8:16] *= 50.0          # eight outlier channels inside one Hadamard block
    errs, theory = _errors(x, d, h, bits)
    assert errs["block_rht"] > 2.0 * errs["rpbh"], errs
    assert errs["dense"] < errs["rpbh"], errs
    assert abs(errs["dense"] / theory - 1.0) < 0.03, (errs, theory)


def test_rotations_agree_without_outliers():
    d, h, bits = 1024, 64, 4
    rng = np.random.default_rng(1)
    x = rng.standard_normal((256, d))
    errs, theory = _errors(x, d, h, bits)
    for k, e in errs.items():
        assert abs(e / theory - 1.0) < 0.05, (k, errs, theory)


@pytest.mark.parametrize("d,h", [(256, 64), (1024, 256), (3072, 256)])
def test_folded_permutation_gives_the_same_rotation(d, h):
    # R x = B D P x, and P x is x[perm]: a producer whose output channels are
    # reordered by perm hands over x[perm] directly, and the rotation of it
    # with the identity permutation and the same signs is the same vector, bit
    # for bit (the same numbers enter the same butterflies).  The elementwise
    # GELU between the two layers keeps the order.
    rng = np.random.default_rng(d + h)
    perm, sign = rpbh.build_rpbh(d, h, 5)
    y = rng.standard_normal((7, d)) * 3.0
    x = quant.gelu_erf(y)
    folded = quant.gelu_erf(y[:, perm])
    np.testing.assert_array_equal(folded, x[:, perm])
    a = rpbh.rotate(x, perm, sign, h)
    b = rpbh.rotate(folded, np.arange(d), sign, h)
    np.testing.assert_array_equal(a, b)
    # and it is not the identity rotation with the same signs on the unfolded vector
    assert not np.allclose(a, rpbh.rotate(x, np.arange(d), sign, h))
