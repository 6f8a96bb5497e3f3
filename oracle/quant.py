"""Weight / activation quantization, index packing and the dequantized
product, fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Method ("OrbitQuant: data-agnostic quantization for image and video",
rcap.io summary, offline and online pseudo-code), in this module's terms:
with R the orthogonal rotation of input dimension d and c_0 < ... < c_{L-1}
the levels of the codebook for d,

* a weight row w (offline) becomes its norm n = |R w| and the index vector
  q(R w / n), where q(v)_k is the index of the level nearest to v_k;
* a token x (online) becomes s = |R x| and q(R x / (s + eps));
* R^T R = I, so R w . R x = w . x (same page, "rotation cancels"
  paragraph) and the layer output is the dot product of the two dequantized
  vectors, n c[q_w] . s c[q_x], taken in the rotated basis.  The page
  measures exactly this as dequantize-then-matmul ("fake quantization",
  caveats paragraph); here it is computed in fp64.

Readings:

* nearest centroid = count of thresholds strictly below u, thresholds being
  midpoints of adjacent centroids; a tie u == theta_j takes the lower
  centroid (the first index of argmin |u - c|).
* eps = 1e-12 (unvalued on the page), added to the norm; the stored scale
  is s itself.  The same guard divides weight rows by (n + eps).
* the codebook is for d = d_in (one codebook per input dimension), not h.
* index 0 is the most negative centroid; packing is row-major, K-contiguous,
  least-significant bits first: a row is a little-endian bit stream, index k
  in bits [k b, (k+1) b) (for 2, 4, 8 bits: LSB first within each byte; the
  pages name 3- and 6-bit widths without a layout, this is its plainest
  extension).
* GELU for the MLP chain is the exact erf form, 0.5 y (1 + erf(y / sqrt 2)).
"""

from __future__ import annotations

import numpy as np
from scipy import special

from .rpbh import rotate

EPS = 1e-12


def nearest_index(u: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """idx = #{j : theta_j < u} (searchsorted with side='left' is that count)."""
    return np.searchsorted(np.asarray(thresholds, dtype=np.float64), u, side="left").astype(np.int64)


def quantize_activations(X, perm, sign, h, thresholds, eps: float = EPS):
    """Online step per token: returns (idx[T, d], s[T], x_rot[T, d], u[T, d])."""
    x_rot = rotate(X, perm, sign, h)
    s = np.linalg.norm(x_rot, axis=1)
    u = x_rot / (s + eps)[:, None]
    return nearest_index(u, thresholds), s, x_rot, u


def quantize_rotated(x_rot, thresholds, eps: float = EPS):
    """The same norm / normalise / nearest-centroid step for rows already
    rotated by any orthogonal R (the dense reference rotation of the page's
    RPBH paragraph, or a variant): returns (idx[T, d], s[T])."""
    s = np.linalg.norm(x_rot, axis=1)
    return nearest_index(x_rot / (s + eps)[:, None], thresholds), s


def relative_error(x_rot, idx, s, centroids) -> float:
    """||s c[idx] - x_rot||_F / ||x_rot||_F: the quantization error of the
    rows; R is orthogonal, so it is also the error in the original basis."""
    xq = np.asarray(s)[:, None] * np.asarray(centroids)[idx]
    return float(np.linalg.norm(xq - x_rot) / np.linalg.norm(x_rot))


def quantize_weights(W, perm, sign, h, thresholds, eps: float = EPS):
    """Offline step per weight matrix: returns (idx[N, d], norms[N], W_rot, u)."""
    w_rot = rotate(W, perm, sign, h)
    n = np.linalg.norm(w_rot, axis=1)
    u = w_rot / (n + eps)[:, None]
    return nearest_index(u, thresholds), n, w_rot, u


def pack(idx: np.ndarray, bits: int) -> np.ndarray:
    """Pack [R, K] indices (< 2^bits, 1 <= bits <= 8) into [R, K*bits/8]
    bytes: each row is a little-endian bit stream in which index k occupies
    bits [k*bits, (k+1)*bits) and byte j holds bits [8j, 8j+8).  For 2, 4
    and 8 bits this is "LSB first within each byte"."""
    idx = np.asarray(idx, dtype=np.int64)
    R, K = idx.shape
    if not 1 <= bits <= 8 or (K * bits) % 8:
        raise ValueError("need 1 <= bits <= 8 and K * bits a whole number of bytes")
    if idx.size and (idx.min() < 0 or idx.max() >= (1 << bits)):
        raise ValueError("index out of range")
    stream = ((idx[:, :, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(R, K * bits)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack`."""
    p = np.asarray(packed, dtype=np.uint8)
    R = p.shape[0]
    stream = np.unpackbits(p, axis=1, bitorder="little")[:, :K * bits].astype(np.int64)
    return (stream.reshape(R, K, bits) << np.arange(bits)).sum(axis=2)


def gelu_erf(y):
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + special.erf(y / np.sqrt(2.0)))


def dequantized_product(ia, s, iw, n, c_a, c_w, bias=None, gelu: bool = False):
    """y = (s * C_a[ia]) @ (n * C_w[iw]).T (+ bias) (GELU), in fp64.

    ia[T, K], s[T] give x_hat; iw[N, K], n[N] give W_hat (both in the rotated
    basis, where the rotation has cancelled).
    """
    x_hat = np.asarray(s, dtype=np.float64)[:, None] * np.asarray(c_a, dtype=np.float64)[ia]
    w_hat = np.asarray(n, dtype=np.float64)[:, None] * np.asarray(c_w, dtype=np.float64)[iw]
    y = x_hat @ w_hat.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if gelu:
        y = gelu_erf(y)
    return y


def boundary_distance(u: np.ndarray, thresholds: np.ndarray):
    """For each u: (|u - theta*|, theta*) for the threshold theta* nearest u."""
    th = np.asarray(thresholds, dtype=np.float64)
    j = np.searchsorted(th, u, side="left")
    lo = th[np.clip(j - 1, 0, len(th) - 1)]
    hi = th[np.clip(j, 0, len(th) - 1)]
    dlo = np.abs(u - lo)
    dhi = np.abs(u - hi)
    near = np.where(dlo <= dhi, lo, hi)
    return np.minimum(dlo, dhi), near
