"""INT4 round-to-nearest weight-only quantization and the W4A16 linear of the
AdaLN modulation projections, fp64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Method: the modulation projections of the adaptive layer norm produce a
timestep-dependent scale and shift, so the rotation trick does not apply to
them and they are kept at INT4 weight round-to-nearest while every other
projection of the block is OrbitQuant-quantized ("OrbitQuant: data-agnostic
quantization for image and video", rcap.io summary: the deployment paragraph
and the AdaLN caveat; the "FLUX.3 Image Klein OrbitQuant W4A8" model card,
Components table: INT4 for the modulation projections).

The pages say no more than "INT4 weight round-to-nearest". Readings (the
plainest scheme that name covers):

* symmetric and signed: codes q in [-8, 7]; one scale per output row and
  group of ``group`` consecutive input columns (group = d_in is per output
  channel), s = max |w| / 7 over the group, rounded to fp32;
* q = clamp(round_half_even(w / s), -8, 7), the division taken in fp64 with
  the stored fp32 scale, so that w_hat = s q uses the same s;
  an all-zero group has s = 0 and q = 0;
* the layer: y[t, o] = sum_g s[o, g] sum_{k in g} q[o, k] x[t, k] (+ bias[o]),
  with x the 16-bit activations as given (weight-only quantization);
* packing: two's-complement nibbles, code k of a row in bits [4k, 4k + 4) of
  the row read as a little-endian bit stream (the layout of the codebook
  indices at 4 bits).
"""

from __future__ import annotations

import numpy as np

QMIN, QMAX = -8, 7


def quantize_int4_rtn(W, group: int):
    """W[N, K] (float) -> (q[N, K] int8 in [-8, 7], scale[N, K // group] fp32)."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide d_in")
    G = K // group
    Wg = W.reshape(N, G, group)
    amax = np.abs(Wg).max(axis=2)                       # [N, G]
    scale = (amax / 7.0).astype(np.float32)             # fp64 division, rounded to fp32
    s64 = scale.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s64 > 0, Wg / np.where(s64 > 0, s64, 1.0), 0.0)
    q = np.clip(np.rint(r), QMIN, QMAX).astype(np.int8)   # rint: round half to even
    return q.reshape(N, K), scale


def dequantize(q, scale, group: int):
    """w_hat[N, K] = s q in fp64."""
    q = np.asarray(q, dtype=np.float64)
    N, K = q.shape
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    return s * q


def linear_w4a16(x, q, scale, group: int, bias=None):
    """y[T, N] = x @ w_hat.T (+ bias), fp64."""
    y = np.asarray(x, dtype=np.float64) @ dequantize(q, scale, group).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def pack_int4(q) -> np.ndarray:
    """[N, K] codes in [-8, 7] -> [N, K / 2] bytes, two's-complement nibbles,
    code k in bits [4k, 4k + 4) of the row's little-endian bit stream."""
    q = np.asarray(q)
    if q.shape[1] % 2:
        raise ValueError("d_in must be even")
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed, K: int) -> np.ndarray:
    """Inverse of :func:`pack_int4`."""
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.empty((p.shape[0], K), dtype=np.int16)
    nib[:, 0::2] = p & 0xF
    nib[:, 1::2] = p >> 4
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)
