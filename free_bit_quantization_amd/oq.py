"""Python binding of liboq (include/oq.h): argument marshalling only.

Every step of the quantized linear runs inside liboq's HIP kernels; this
module only turns torch tensors into device pointers and HIP stream handles
(torch provides device memory and streams), allocates outputs with torch
when the caller does not pass them, and turns status codes into exceptions.
There is no fallback: if liboq.so is missing or a call fails, it raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboq.so")

OQ_OK, OQ_EINVAL, OQ_EUNSUPPORTED, OQ_ENOCONV, OQ_EDEVICE = 0, -1, -2, -3, -4
OQ_F32, OQ_BF16, OQ_F16 = 0, 1, 2
OQ_EPI_NONE, OQ_EPI_GELU_ERF, OQ_EPI_OUT_BF16 = 0, 1, 0x100

# every symbol include/oq.h declares
EXPORTS = ("oq_last_error", "oq_version", "oq_build_rpbh", "oq_build_block_rht", "oq_lloyd_max",
           "oq_quantize_weights", "oq_rotate_quantize_act", "oq_qlinear", "oq_quantize_weights_int4",
           "oq_linear_w4a16")


class OQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"liboq status {status}: {msg}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)


def lib() -> ctypes.CDLL:
    """Load liboq.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.oq_last_error.restype = ctypes.c_char_p
        L.oq_last_error.argtypes = []
        L.oq_version.restype = ctypes.c_char_p
        L.oq_version.argtypes = []
        L.oq_build_rpbh.restype = _I32
        L.oq_build_rpbh.argtypes = [_I32, _I32, ctypes.c_uint64, _P, _P]
        L.oq_build_block_rht.restype = _I32
        L.oq_build_block_rht.argtypes = [_I32, _I32, ctypes.c_uint64, _P, _P]
        L.oq_lloyd_max.restype = _I32
        L.oq_lloyd_max.argtypes = [_I32, _I32, _P, _P, _P]
        L.oq_quantize_weights.restype = _I32
        L.oq_quantize_weights.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P]
        L.oq_rotate_quantize_act.restype = _I32
        L.oq_rotate_quantize_act.argtypes = [_P, _I32, _I64, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _P]
        L.oq_qlinear.restype = _I32
        L.oq_qlinear.argtypes = [_P, _P, _I64, _P, _P, _I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P, _P]
        L.oq_quantize_weights_int4.restype = _I32
        L.oq_quantize_weights_int4.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P]
        L.oq_linear_w4a16.restype = _I32
        L.oq_linear_w4a16.argtypes = [_P, _I32, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P]
        _lib = L
    return _lib


def _check(status: int):
    if status != OQ_OK:
        raise OQError(status, lib().oq_last_error().decode())


def _host_f64(a) -> Tuple[np.ndarray, int]:
    arr = np.ascontiguousarray(a, dtype=np.float64)
    return arr, arr.ctypes.data


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


# ---------------------------------------------------------------------------
# host calls
# ---------------------------------------------------------------------------


def oq_version() -> str:
    return lib().oq_version().decode()


def oq_build_rpbh(d: int, h: int, seed: int = 0):
    """(perm int32[d], sign int8[d]) of the seeded RPBH rotation."""
    perm = np.empty(d, dtype=np.int32)
    sign = np.empty(d, dtype=np.int8)
    _check(lib().oq_build_rpbh(d, h, seed, perm.ctypes.data, sign.ctypes.data))
    return perm, sign


def oq_build_block_rht(d: int, h: int, seed: int = 0):
    """(perm int32[d] = identity, sign int8[d]) of the Block-RHT ablation variant."""
    perm = np.empty(d, dtype=np.int32)
    sign = np.empty(d, dtype=np.int8)
    _check(lib().oq_build_block_rht(d, h, seed, perm.ctypes.data, sign.ctypes.data))
    return perm, sign


def oq_lloyd_max(d: int, bits: int):
    """(centroids[2^bits], thresholds[2^bits - 1], mse) for the marginal f_d."""
    L = 1 << bits
    c = np.empty(L, dtype=np.float64)
    th = np.empty(L - 1, dtype=np.float64)
    mse = ctypes.c_double(0.0)
    _check(lib().oq_lloyd_max(d, bits, c.ctypes.data, th.ctypes.data, ctypes.addressof(mse)))
    return c, th, mse.value


# ---------------------------------------------------------------------------
# device calls (torch tensors on the current device)
# ---------------------------------------------------------------------------


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return OQ_F32
    if t.dtype == torch.bfloat16:
        return OQ_BF16
    raise TypeError("expected float32 or bfloat16")


def oq_quantize_weights(W, h: int, perm, sign, thresholds, bits_w: int, w_idx=None, w_norm=None, stream=None):
    """Offline weight step: returns (w_idx uint8[d_out, d_in*bits/8], w_norm f32[d_out])."""
    import torch
    d_out, d_in = W.shape
    if w_idx is None:
        w_idx = torch.empty((d_out, d_in * bits_w // 8), dtype=torch.uint8, device=W.device)
    if w_norm is None:
        w_norm = torch.empty(d_out, dtype=torch.float32, device=W.device)
    th, thp = _host_f64(thresholds)
    _check(lib().oq_quantize_weights(_dev(W), _dtype_code(W), d_out, d_in, h, _dev(perm, torch.int32),
                                     _dev(sign, torch.int8), thp, bits_w, _dev(w_idx, torch.uint8),
                                     _dev(w_norm, torch.float32), _stream(stream)))
    return w_idx, w_norm


def oq_rotate_quantize_act(x, h: int, perm, sign, thresholds, bits_a: int, x_idx=None, s=None,
                           x_rot: Optional[object] = None, want_x_rot: bool = False, stream=None):
    """Online activation step: returns (x_idx uint8[T, d*bits/8], s f32[T], x_rot f32[T, d] or None)."""
    import torch
    T, d = x.shape
    if x_idx is None:
        x_idx = torch.empty((T, d * bits_a // 8), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(T, dtype=torch.float32, device=x.device)
    if x_rot is None and want_x_rot:
        x_rot = torch.empty((T, d), dtype=torch.float32, device=x.device)
    th, thp = _host_f64(thresholds)
    _check(lib().oq_rotate_quantize_act(_dev(x), _dtype_code(x), T, d, h, _dev(perm, torch.int32),
                                        _dev(sign, torch.int8), thp, bits_a, _dev(x_idx, torch.uint8),
                                        _dev(s, torch.float32),
                                        _dev(x_rot, torch.float32) if x_rot is not None else None,
                                        _stream(stream)))
    return x_idx, s, x_rot


def oq_qlinear(x_idx, s, w_idx, w_norm, d_in: int, centroids_a, bits_a: int, centroids_w, bits_w: int,
               bias=None, epilogue: int = OQ_EPI_NONE, y=None, stream=None, out_dtype=None):
    """Codebook GEMM: returns y[T, d_out], float32 (default) or bfloat16
    (out_dtype=torch.bfloat16, or a bf16 y: the fp32 result rounded to nearest even)."""
    import torch
    T = s.shape[0]
    d_out = w_norm.shape[0]
    if y is None:
        y = torch.empty((T, d_out), dtype=out_dtype or torch.float32, device=s.device)
    if y.dtype == torch.bfloat16:
        epilogue |= OQ_EPI_OUT_BF16
    elif y.dtype != torch.float32:
        raise TypeError("y must be float32 or bfloat16")
    ca, cap = _host_f64(centroids_a)
    cw, cwp = _host_f64(centroids_w)
    _check(lib().oq_qlinear(_dev(x_idx, torch.uint8), _dev(s, torch.float32), T, _dev(w_idx, torch.uint8),
                            _dev(w_norm, torch.float32), d_out, d_in, cap, bits_a, cwp, bits_w,
                            _dev(bias, torch.float32) if bias is not None else None, epilogue,
                            _dev(y, y.dtype), _stream(stream)))
    return y


def oq_quantize_weights_int4(W, group: int, q=None, scale=None, stream=None):
    """INT4 round-to-nearest weights (AdaLN modulation): returns
    (q uint8[d_out, d_in/2], scale f32[d_out, d_in/group])."""
    import torch
    d_out, d_in = W.shape
    if q is None:
        q = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((d_out, d_in // group), dtype=torch.float32, device=W.device)
    _check(lib().oq_quantize_weights_int4(_dev(W), _dtype_code(W), d_out, d_in, group, _dev(q, torch.uint8),
                                          _dev(scale, torch.float32), _stream(stream)))
    return q, scale


def oq_linear_w4a16(x, q, scale, group: int, bias=None, y=None, stream=None):
    """W4A16 product with INT4 RTN weights: returns y f32[T, d_out]; x is bf16 or fp16."""
    import torch
    T, d_in = x.shape
    d_out = q.shape[0]
    if x.dtype == torch.bfloat16:
        code = OQ_BF16
    elif x.dtype == torch.float16:
        code = OQ_F16
    else:
        raise TypeError("x must be bfloat16 or float16")
    if y is None:
        y = torch.empty((T, d_out), dtype=torch.float32, device=x.device)
    _check(lib().oq_linear_w4a16(_dev(x), code, T, _dev(q, torch.uint8), _dev(scale, torch.float32), d_out, d_in,
                                 group, _dev(bias, torch.float32) if bias is not None else None,
                                 _dev(y, torch.float32), _stream(stream)))
    return y
