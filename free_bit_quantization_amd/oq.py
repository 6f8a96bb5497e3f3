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
           "oq_quantize_weights", "oq_rotate_quantize_act", "oq_qlinear", "oq_qlinear_workspace_size",
           "oq_qlinear_splitk", "oq_qlinear_splitk_noalloc", "oq_fold_permutation", "oq_quantize_weights_int4",
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
        L.oq_qlinear_workspace_size.restype = _I32
        L.oq_qlinear_workspace_size.argtypes = [_I64, _I32, _I32, _I32, _I32, _P]
        L.oq_qlinear_splitk.restype = _I32
        L.oq_qlinear_splitk.argtypes = [_P, _P, _I64, _P, _P, _I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P, _P,
                                        ctypes.c_size_t, _P]
        L.oq_qlinear_splitk_noalloc.restype = _I32
        L.oq_qlinear_splitk_noalloc.argtypes = [_P, _P, _I64, _P, _P, _I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P, _P]
        L.oq_fold_permutation.restype = _I32
        L.oq_fold_permutation.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]
        L.oq_quantize_weights_int4.restype = _I32
        L.oq_quantize_weights_int4.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P]
        L.oq_linear_w4a16.restype = _I32
        L.oq_linear_w4a16.argtypes = [_P, _I32, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P]
        _lib = L
    return _lib


def _check(status: int):
    if status != OQ_OK:
        raise OQError(status, lib().oq_last_error().decode())


def _host_f64(a, n: Optional[int] = None, what: str = "table") -> Tuple[np.ndarray, int]:
    """A contiguous float64 host copy of a table (length n if given: the
    library reads exactly that many entries)."""
    arr = np.ascontiguousarray(a, dtype=np.float64)
    if arr.ndim != 1 or (n is not None and arr.shape[0] != n):
        raise ValueError(f"{what} must be a 1-D array of {n} values (got shape {arr.shape})")
    return arr, arr.ctypes.data


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _meta(t, dtype=None, shape=None, what: str = "tensor"):
    """Check a tensor's shape and dtype (device not yet)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    return t


def _dev(t, dtype=None, shape=None, what: str = "tensor"):
    """Device pointer of a contiguous tensor on the current HIP device, after
    checking its shape, dtype and device."""
    import torch
    _meta(t, dtype, shape, what)
    if not t.is_cuda:
        raise TypeError(f"{what}: expected a device (cuda) tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _packed_cols(d: int, bits: int, what: str) -> int:
    if (d * bits) % 8 != 0:
        raise ValueError(f"{what}: d * bits must fill whole bytes (d={d}, bits={bits})")
    return d * bits // 8


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
    cols = _packed_cols(d_in, bits_w, "w_idx")
    th, thp = _host_f64(thresholds, (1 << bits_w) - 1, "thresholds")
    _meta(perm, torch.int32, (d_in,), "perm")
    _meta(sign, torch.int8, (d_in,), "sign")
    pp = _dev(perm, torch.int32, (d_in,), "perm")
    sp = _dev(sign, torch.int8, (d_in,), "sign")
    if w_idx is None:
        w_idx = torch.empty((d_out, cols), dtype=torch.uint8, device=W.device)
    if w_norm is None:
        w_norm = torch.empty(d_out, dtype=torch.float32, device=W.device)
    _check(lib().oq_quantize_weights(_dev(W, what="W"), _dtype_code(W), d_out, d_in, h, pp, sp, thp, bits_w,
                                     _dev(w_idx, torch.uint8, (d_out, cols), "w_idx"),
                                     _dev(w_norm, torch.float32, (d_out,), "w_norm"), _stream(stream)))
    return w_idx, w_norm


def oq_fold_permutation(w_idx, w_norm, perm_next, d_in: int, bits_w: int, bias=None, stream=None):
    """Offline: this layer's quantized rows reordered by the next layer's RPBH
    permutation (out[i] = in[perm_next[i]]): returns (w_idx, w_norm, bias or
    None), new tensors.  The next rotate-quantize of GELU(y) then takes the
    identity permutation with its own signs."""
    import torch
    d_out = w_norm.shape[0]
    cols = _packed_cols(d_in, bits_w, "w_idx")
    _meta(w_idx, torch.uint8, (d_out, cols), "w_idx")
    _meta(w_norm, torch.float32, (d_out,), "w_norm")
    _meta(perm_next, torch.int32, (d_out,), "perm_next")
    if bias is not None:
        _meta(bias, torch.float32, (d_out,), "bias")
    wi = torch.empty_like(w_idx)
    wn = torch.empty_like(w_norm)
    bo = torch.empty_like(bias) if bias is not None else None
    _check(lib().oq_fold_permutation(_dev(w_idx, what="w_idx"), _dev(w_norm, what="w_norm"),
                                     _dev(bias, what="bias") if bias is not None else None, d_out, d_in, bits_w,
                                     _dev(perm_next, what="perm_next"), _dev(wi, what="w_idx_out"),
                                     _dev(wn, what="w_norm_out"), _dev(bo, what="bias_out") if bo is not None else None,
                                     _stream(stream)))
    return wi, wn, bo


def oq_rotate_quantize_act(x, h: int, perm, sign, thresholds, bits_a: int, x_idx=None, s=None,
                           x_rot: Optional[object] = None, want_x_rot: bool = False, stream=None):
    """Online activation step: returns (x_idx uint8[T, d*bits/8], s f32[T], x_rot f32[T, d] or None)."""
    import torch
    T, d = x.shape
    cols = _packed_cols(d, bits_a, "x_idx")
    th, thp = _host_f64(thresholds, (1 << bits_a) - 1, "thresholds")
    _meta(perm, torch.int32, (d,), "perm")
    _meta(sign, torch.int8, (d,), "sign")
    pp = _dev(perm, torch.int32, (d,), "perm")
    sp = _dev(sign, torch.int8, (d,), "sign")
    if x_idx is None:
        x_idx = torch.empty((T, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(T, dtype=torch.float32, device=x.device)
    if x_rot is None and want_x_rot:
        x_rot = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _check(lib().oq_rotate_quantize_act(_dev(x, what="x"), _dtype_code(x), T, d, h, pp, sp, thp, bits_a,
                                        _dev(x_idx, torch.uint8, (T, cols), "x_idx"),
                                        _dev(s, torch.float32, (T,), "s"),
                                        _dev(x_rot, torch.float32, (T, d), "x_rot") if x_rot is not None else None,
                                        _stream(stream)))
    return x_idx, s, x_rot


def _qlinear_args(x_idx, s, w_idx, w_norm, d_in, centroids_a, bits_a, centroids_w, bits_w, bias, epilogue, y,
                  out_dtype):
    """Checked arguments shared by the GEMM entry points (y allocated if None)."""
    import torch
    T = s.shape[0]
    d_out = w_norm.shape[0]
    ca, cap = _host_f64(centroids_a, 1 << bits_a, "centroids_a")
    cw, cwp = _host_f64(centroids_w, 1 << bits_w, "centroids_w")
    # shapes and dtypes of every operand first, then their devices
    _meta(x_idx, torch.uint8, (T, _packed_cols(d_in, bits_a, "x_idx")), "x_idx")
    _meta(s, torch.float32, (T,), "s")
    _meta(w_idx, torch.uint8, (d_out, _packed_cols(d_in, bits_w, "w_idx")), "w_idx")
    _meta(w_norm, torch.float32, (d_out,), "w_norm")
    if bias is not None:
        _meta(bias, torch.float32, (d_out,), "bias")
    if y is not None:
        _meta(y, None, (T, d_out), "y")
    xi = _dev(x_idx, torch.uint8, (T, _packed_cols(d_in, bits_a, "x_idx")), "x_idx")
    sp = _dev(s, torch.float32, (T,), "s")
    wi = _dev(w_idx, torch.uint8, (d_out, _packed_cols(d_in, bits_w, "w_idx")), "w_idx")
    wn = _dev(w_norm, torch.float32, (d_out,), "w_norm")
    bp = _dev(bias, torch.float32, (d_out,), "bias") if bias is not None else None
    if y is None:
        y = torch.empty((T, d_out), dtype=out_dtype or torch.float32, device=s.device)
    if y.dtype == torch.bfloat16:
        epilogue |= OQ_EPI_OUT_BF16
    elif y.dtype != torch.float32:
        raise TypeError("y must be float32 or bfloat16")
    args = (xi, sp, T, wi, wn, d_out, d_in, cap, bits_a, cwp, bits_w, bp, epilogue, _dev(y, y.dtype, (T, d_out), "y"))
    return y, args, (ca, cw)


def oq_qlinear(x_idx, s, w_idx, w_norm, d_in: int, centroids_a, bits_a: int, centroids_w, bits_w: int,
               bias=None, epilogue: int = OQ_EPI_NONE, y=None, stream=None, out_dtype=None):
    """Codebook GEMM (whole tiles, no workspace): returns y[T, d_out], float32
    (default) or bfloat16 (out_dtype=torch.bfloat16, or a bf16 y: the fp32
    result rounded to nearest even)."""
    y, args, _keep = _qlinear_args(x_idx, s, w_idx, w_norm, d_in, centroids_a, bits_a, centroids_w, bits_w, bias,
                                   epilogue, y, out_dtype)
    _check(lib().oq_qlinear(*args, _stream(stream)))
    return y


def oq_qlinear_workspace_size(T: int, d_out: int, d_in: int, bits_a: int, bits_w: int) -> int:
    """Bytes of workspace oq_qlinear_splitk needs for this shape on the current device (0: no split)."""
    n = ctypes.c_size_t(0)
    _check(lib().oq_qlinear_workspace_size(T, d_out, d_in, bits_a, bits_w, ctypes.addressof(n)))
    return n.value


def qlinear_workspace(T: int, d_out: int, d_in: int, bits_a: int, bits_w: int, device=None):
    """A zero-filled workspace for oq_qlinear_splitk (a uint8 tensor, allocated
    by torch), or None when the shape takes no split."""
    import torch
    n = oq_qlinear_workspace_size(T, d_out, d_in, bits_a, bits_w)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


def oq_qlinear_splitk(x_idx, s, w_idx, w_norm, d_in: int, centroids_a, bits_a: int, centroids_w, bits_w: int,
                      workspace, bias=None, epilogue: int = OQ_EPI_NONE, y=None, stream=None, out_dtype=None):
    """Codebook GEMM with the last partial round of tiles split along K
    (stream-K) through a caller-owned workspace (from qlinear_workspace, or
    None when the shape takes no split)."""
    import torch
    y, args, _keep = _qlinear_args(x_idx, s, w_idx, w_norm, d_in, centroids_a, bits_a, centroids_w, bits_w, bias,
                                   epilogue, y, out_dtype)
    if workspace is None:
        wp, wn = None, 0
    else:
        wp, wn = _dev(workspace, torch.uint8, what="workspace"), workspace.numel()
    _check(lib().oq_qlinear_splitk(*args, wp, wn, _stream(stream)))
    return y


def oq_qlinear_splitk_noalloc(x_idx, s, w_idx, w_norm, d_in: int, centroids_a, bits_a: int, centroids_w,
                              bits_w: int, bias=None, epilogue: int = OQ_EPI_NONE, y=None, stream=None,
                              out_dtype=None):
    """oq_qlinear_splitk through the library's own device scratch (no
    workspace argument; calls on one device must not overlap).  Allocates
    y only when it is not given."""
    y, args, _keep = _qlinear_args(x_idx, s, w_idx, w_norm, d_in, centroids_a, bits_a, centroids_w, bits_w, bias,
                                   epilogue, y, out_dtype)
    _check(lib().oq_qlinear_splitk_noalloc(*args, _stream(stream)))
    return y


def oq_quantize_weights_int4(W, group: int, q=None, scale=None, stream=None):
    """INT4 round-to-nearest weights (AdaLN modulation): returns
    (q uint8[d_out, d_in/2], scale f32[d_out, d_in/group])."""
    import torch
    d_out, d_in = W.shape
    if group <= 0 or d_in % group != 0 or d_in % 2 != 0:
        raise ValueError(f"group ({group}) must divide d_in ({d_in}), d_in even")
    if q is None:
        q = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=W.device)
    if scale is None:
        scale = torch.empty((d_out, d_in // group), dtype=torch.float32, device=W.device)
    _check(lib().oq_quantize_weights_int4(_dev(W, what="W"), _dtype_code(W), d_out, d_in, group,
                                          _dev(q, torch.uint8, (d_out, d_in // 2), "q"),
                                          _dev(scale, torch.float32, (d_out, d_in // group), "scale"),
                                          _stream(stream)))
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
    if group <= 0 or d_in % group != 0:
        raise ValueError(f"group ({group}) must divide d_in ({d_in})")
    if y is None:
        y = torch.empty((T, d_out), dtype=torch.float32, device=x.device)
    _check(lib().oq_linear_w4a16(_dev(x, what="x"), code, T, _dev(q, torch.uint8, (d_out, d_in // 2), "q"),
                                 _dev(scale, torch.float32, (d_out, d_in // group), "scale"), d_out, d_in, group,
                                 _dev(bias, torch.float32, (d_out,), "bias") if bias is not None else None,
                                 _dev(y, torch.float32, (T, d_out), "y"), _stream(stream)))
    return y
