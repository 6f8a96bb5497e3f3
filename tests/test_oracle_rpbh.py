"""Pins of the oracle's RPBH rotation against what the pages and the
mathematics fix (orthogonality, fast = dense, cancellation, uniformity,
the published splitmix64 vectors)."""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import rpbh


def _shapes(max_d=256):
    out = []
    for d in (2, 8, 64, 96, 256):
        if d > max_d:
            continue
        h = 2
        while h <= d:
            if d % h == 0:
                out.append((d, h))
            h *= 2
    return out


def test_splitmix64_published_vectors(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "splitmix64.json")))
    for v in g["vectors"]:
        r = rpbh.SplitMix64(v["seed"])
        assert [r.next() for _ in v["outputs"]] == [int(x) for x in v["outputs"]]


def test_sylvester_construction():
    # Sylvester's recursion H_2n = [[H, H], [H, -H]] from H_1 = [1]
    H = np.array([[1.0]])
    for m in range(1, 9):
        H = np.block([[H, H], [H, -H]])
        np.testing.assert_array_equal(rpbh.sylvester(2 ** m), H)
    assert np.allclose(H @ H.T, 256 * np.eye(256))


@pytest.mark.parametrize("d,h", _shapes())
def test_rotation_orthogonal(d, h):
    perm, sign = rpbh.build_rpbh(d, h, seed=7)
    R = rpbh.dense_rotation(perm, sign, h)
    assert np.max(np.abs(R @ R.T - np.eye(d))) <= 1e-15 * 4


@pytest.mark.parametrize("d,h", _shapes())
def test_fast_equals_dense(d, h):
    perm, sign = rpbh.build_rpbh(d, h, seed=3)
    R = rpbh.dense_rotation(perm, sign, h)
    X = np.random.default_rng(1).standard_normal((5, d))
    fast = rpbh.rotate(X, perm, sign, h)
    dense = X @ R.T
    assert np.max(np.abs(fast - dense)) <= 1e-14 * np.max(np.abs(dense))


def test_dense_rotation_is_block_hadamard_of_signed_gather():
    # independent brute force of R = B D P for one small case, entry by entry
    d, h = 8, 4
    perm, sign = rpbh.build_rpbh(d, h, seed=11)
    R = rpbh.dense_rotation(perm, sign, h)
    for i in range(d):
        for k in range(d):
            blk_i, blk_k = i // h, k // h
            want = 0.0
            # (B D P)[i, k] = sum_j B[i, j] sign[j] [perm[j] == k]
            for j in range(blk_i * h, blk_i * h + h):
                if perm[j] == k:
                    a, b = i % h, j % h
                    want += (-1) ** bin(a & b).count("1") / np.sqrt(h) * sign[j]
            assert abs(R[i, k] - want) < 1e-15
            del blk_k


def test_rotation_cancels_in_layer():
    d, h, n = 256, 64, 40
    perm, sign = rpbh.build_rpbh(d, h, seed=0)
    rng = np.random.default_rng(2)
    W = rng.standard_normal((n, d))
    x = rng.standard_normal((9, d))
    w_rot = rpbh.rotate(W, perm, sign, h)       # W @ R.T
    x_rot = rpbh.rotate(x, perm, sign, h)       # x @ R.T
    y_rot = x_rot @ w_rot.T                      # (R x) . (R w)
    y = x @ W.T
    assert np.max(np.abs(y_rot - y)) <= 1e-13 * np.max(np.abs(y))


def test_perm_bijection_signs_deterministic():
    perm, sign = rpbh.build_rpbh(3072, 256, 0)
    assert sorted(perm.tolist()) == list(range(3072))
    assert set(sign.tolist()) == {-1, 1}
    p2, s2 = rpbh.build_rpbh(3072, 256, 0)
    assert np.array_equal(perm, p2) and np.array_equal(sign, s2)
    p3, _ = rpbh.build_rpbh(3072, 256, 1)
    assert not np.array_equal(perm, p3)
    # the balance of the signs is that of fair coin flips
    assert abs(int(sign.sum())) < 5 * np.sqrt(3072)


def test_perm_uniform_chi2():
    # "uniform random permutation": perm[0] over many seeds is uniform on 0..7,
    # and so is the position of element 0
    d, n = 8, 20000
    c0 = np.zeros(d)
    cpos = np.zeros(d)
    for s in range(n):
        p, _ = rpbh.build_rpbh(d, 2, s)
        c0[p[0]] += 1
        cpos[int(np.where(p == 0)[0][0])] += 1
    assert stats.chisquare(c0).pvalue > 1e-3
    assert stats.chisquare(cpos).pvalue > 1e-3


@pytest.mark.parametrize("d,h", [(0, 2), (8, 3), (8, 16), (12, 8), (8, 1)])
def test_invalid_shapes(d, h):
    with pytest.raises(ValueError):
        rpbh.build_rpbh(d, h, 0)
