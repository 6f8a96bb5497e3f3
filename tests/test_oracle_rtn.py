"""Pins of the INT4 round-to-nearest oracle (AdaLN modulation projections)."""

import json
import os

import numpy as np
import pytest

from oracle import rtn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_rtn_hand.json")


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"])
def test_hand_worked_examples(case):
    w = np.array([case["w"]], dtype=np.float32)
    q, s = rtn.quantize_int4_rtn(w, case["group"])
    np.testing.assert_array_equal(s[0], np.array(case["scale"], dtype=np.float32))
    np.testing.assert_array_equal(q[0], case["q"])
    np.testing.assert_array_equal(rtn.pack_int4(q)[0], case["packed"])
    np.testing.assert_array_equal(rtn.unpack_int4(rtn.pack_int4(q), w.shape[1]), q)


def test_scale_two_sevenths_bits():
    # the hand value of fp32(2/7): mantissa round(2/7 * 2^25) = 9586981
    assert np.float32(2.0 / 7.0) == np.float32(9586981 * 2.0 ** -25)
    assert 9586981 * 2.0 ** -25 > 2.0 / 7.0


@pytest.mark.parametrize("group", [8, 64, 256])
def test_rounding_error_bound_and_extremes(group):
    rng = np.random.default_rng(group)
    W = rng.standard_normal((37, 512)).astype(np.float32) * rng.uniform(0.01, 3.0, (37, 1)).astype(np.float32)
    q, s = rtn.quantize_int4_rtn(W, group)
    assert q.min() >= -8 and q.max() <= 7
    err = np.abs(W.astype(np.float64) - rtn.dequantize(q, s, group))
    bound = np.repeat(s.astype(np.float64), group, axis=1) * (0.5 + 1e-6)
    assert np.all(err <= bound)
    # the largest |w| of every group lands on +-7 exactly
    qg = np.abs(q.reshape(37, -1, group)).max(axis=2)
    assert np.all(qg == 7)
    # -8 is never produced by a symmetric max / 7 scale
    assert q.min() >= -7


def test_uniform_rounding_noise_variance():
    # W ~ U(-1, 1) over 4096 columns: max |w| = 1 - O(1/4096), so s = 1/7 and
    # RTN noise is ~ U(-s/2, s/2), variance (1/7)^2 / 12, fixed by the
    # distribution alone (a divisor of 8 would give (7/8)^2 of it)
    rng = np.random.default_rng(5)
    W = rng.uniform(-1.0, 1.0, (64, 4096))
    q, s = rtn.quantize_int4_rtn(W, 4096)
    e = W - rtn.dequantize(q, s, 4096)
    ratio = np.mean(e ** 2) / ((1.0 / 7.0) ** 2 / 12.0)
    assert abs(ratio - 1.0) < 0.03


def test_degenerate_rows():
    W = np.zeros((3, 16), dtype=np.float32)
    W[1, 5] = -3.0
    W[2, :] = 2.5
    q, s = rtn.quantize_int4_rtn(W, 16)
    assert s[0, 0] == 0 and not q[0].any()
    assert q[1, 5] == -7 and np.count_nonzero(q[1]) == 1 and s[1, 0] == np.float32(3.0 / 7.0)
    assert np.all(q[2] == 7)


def test_scale_equivariance_power_of_two():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((9, 128)).astype(np.float32)
    q1, s1 = rtn.quantize_int4_rtn(W, 32)
    q2, s2 = rtn.quantize_int4_rtn(W * np.float32(8.0), 32)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1 * np.float32(8.0), s2)


def test_nibble_roundtrip_all_codes():
    q = np.arange(-8, 8, dtype=np.int8).reshape(1, 16)
    p = rtn.pack_int4(q)
    np.testing.assert_array_equal(p[0], [0x98, 0xBA, 0xDC, 0xFE, 0x10, 0x32, 0x54, 0x76])
    np.testing.assert_array_equal(rtn.unpack_int4(p, 16), q)


def test_linear_against_bruteforce_loops():
    rng = np.random.default_rng(3)
    T, N, K, g = 2, 3, 8, 4
    x = rng.standard_normal((T, K))
    W = rng.standard_normal((N, K)).astype(np.float32)
    b = rng.standard_normal(N)
    q, s = rtn.quantize_int4_rtn(W, g)
    y = rtn.linear_w4a16(x, q, s, g, bias=b)
    for t in range(T):
        for o in range(N):
            acc = 0.0
            for grp in range(K // g):
                part = 0.0
                for k in range(grp * g, (grp + 1) * g):
                    part += float(q[o, k]) * x[t, k]
                acc += float(s[o, grp]) * part
            assert abs(y[t, o] - (acc + b[o])) <= 1e-12 * (1 + abs(acc))


def test_per_channel_is_one_group():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((5, 64)).astype(np.float32)
    q, s = rtn.quantize_int4_rtn(W, 64)
    assert s.shape == (5, 1)
    np.testing.assert_array_equal(s[:, 0], (np.abs(W.astype(np.float64)).max(axis=1) / 7.0).astype(np.float32))
