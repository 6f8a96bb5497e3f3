"""Randomized Permuted Block-Hadamard (RPBH) rotation, fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Method ("OrbitQuant: data-agnostic quantization for image and video",
rcap.io summary, paragraph on Randomized Permuted Block-Hadamard rotation,
and the offline pseudo-code line that builds ``rotation[d]``): a uniform
random permutation, random sign flips and block-diagonal Walsh-Hadamard
blocks of size h.  The rotation is orthogonal, applied as ``x @ R.T``.

Readings (the page leaves these open):

* order: R = B . D . P -- permute, then flip signs, then the block
  Hadamard.  (P x)_i = x[perm[i]] (a gather over all d coordinates, not
  per block, because the permutation must spread an outlier across
  blocks), D = diag(sign), B = blockdiag(H_h / sqrt(h)).
* H_h is the Sylvester matrix, H[i, j] = (-1)^popcount(i & j), scaled by
  1/sqrt(h) so that R is orthogonal.
* randomness: a splitmix64 stream seeded with ``seed`` (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
  the 64-bit finalizer constants are the published ones).  Fisher-Yates
  from i = d-1 down to 1 with j = floor(next * (i+1) / 2^64), then one
  more draw per coordinate i = 0..d-1 whose top bit set means sign -1.
  Any uniform RNG gives a correct method; fixing this one makes the
  permutation bit-checkable against the library.
"""

from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1


class SplitMix64:
    """splitmix64 as published: add the golden-gamma increment, then mix."""

    GAMMA = 0x9E3779B97F4A7C15

    def __init__(self, seed: int):
        self.state = seed & _MASK64

    def next(self) -> int:
        self.state = (self.state + self.GAMMA) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)


def build_rpbh(d: int, h: int, seed: int):
    """Return (perm, sign): perm[i] is the source coordinate of output i.

    Requires h a power of two with 2 <= h and h | d.
    """
    if d <= 0 or h < 2 or (h & (h - 1)) != 0 or d % h != 0:
        raise ValueError(f"invalid RPBH shape d={d} h={h}")
    rng = SplitMix64(seed)
    perm = list(range(d))
    for i in range(d - 1, 0, -1):
        j = (rng.next() * (i + 1)) >> 64
        perm[i], perm[j] = perm[j], perm[i]
    sign = [(-1 if (rng.next() >> 63) else 1) for _ in range(d)]
    return np.asarray(perm, dtype=np.int64), np.asarray(sign, dtype=np.int8)


def build_block_rht(d: int, h: int, seed: int):
    """Block-RHT, the ablation variant without the leading permutation.

    Same page, ablation paragraph (removing RPBH's uniform permutation).
    Reading: perm is the identity and the signs are the first d draws of the
    same splitmix64 stream (the RPBH sign rule without the shuffle draws).
    """
    if d <= 0 or h < 2 or (h & (h - 1)) != 0 or d % h != 0:
        raise ValueError(f"invalid Block-RHT shape d={d} h={h}")
    rng = SplitMix64(seed)
    sign = [(-1 if (rng.next() >> 63) else 1) for _ in range(d)]
    return np.arange(d, dtype=np.int64), np.asarray(sign, dtype=np.int8)


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """A dense Haar-random orthogonal d x d matrix (fp64): QR of a Gaussian
    matrix with the signs of R's diagonal moved into Q (Mezzadri, "How to
    generate random matrices from the classical compact groups", 2007).

    The page's reference point for RPBH: a dense random rotation, O(d^2) per
    token, which RPBH replaces (paragraph on the RPBH rotation).
    """
    g = np.random.default_rng(np.random.SeedSequence([seed, d]))
    q, r = np.linalg.qr(g.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def sylvester(h: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(h)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def dense_rotation(perm: np.ndarray, sign: np.ndarray, h: int) -> np.ndarray:
    """R = B . D . P as an explicit d x d fp64 matrix (small d only)."""
    d = perm.shape[0]
    P = np.zeros((d, d))
    P[np.arange(d), perm] = 1.0
    D = np.diag(sign.astype(np.float64))
    B = np.kron(np.eye(d // h), sylvester(h) / np.sqrt(h))
    return B @ D @ P


def rotate(X: np.ndarray, perm: np.ndarray, sign: np.ndarray, h: int) -> np.ndarray:
    """x_rot = x @ R.T for every row of X, by the fast transform.

    Gather y_i = sign_i * x[perm_i], then, inside each block of h, log2(h)
    butterfly stages (a, b) -> (a + b, a - b) on index pairs differing in
    one bit, then the 1/sqrt(h) scale.  O(d log h) per row.
    """
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    Y = X[:, perm] * sign.astype(np.float64)
    Y = Y.reshape(T, d // h, h).copy()
    stride = 1
    while stride < h:
        Y = Y.reshape(T, d // h, h // (2 * stride), 2, stride)
        a = Y[:, :, :, 0, :].copy()
        b = Y[:, :, :, 1, :].copy()
        Y[:, :, :, 0, :] = a + b
        Y[:, :, :, 1, :] = a - b
        stride *= 2
    return Y.reshape(T, d) / np.sqrt(h)
