"""Shared helpers of the GPU parity tests: run one linear through liboq and
through the fp64 oracle on the same seeded inputs and compare."""

from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np

from free_bit_quantization_amd import oq, synth
from oracle import codebook, quant, rpbh

REL_XROT = 1e-5       # per-token relative L2 of the rotated activations
REL_S = 1e-5          # relative error of the token norms
REL_GEMM = 2e-3       # relative Frobenius error of the GEMM output
# Indices may differ only within BAND * |theta| of a threshold: the kernels
# decide every coordinate as exact arithmetic would (certified fp32 fast path,
# fp64 recheck against the fp64 threshold), so what is left is the fp64
# rounding of the two sides' different summation orders (< ~1e-12 relative).
BAND = 1e-11


def sample_rows(T, n, seed=0):
    """The first and last 16 rows and n random ones (sorted, distinct)."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(16, T))
    tail = np.arange(max(0, T - 16), T)
    mid = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Codebooks:
    c: np.ndarray
    th: np.ndarray


_cb_cache = {}


def library_codebook(d: int, bits: int) -> Codebooks:
    """The library's codebook, checked against the oracle's own Lloyd-Max solve."""
    key = (d, bits)
    if key not in _cb_cache:
        c, th, _ = oq.oq_lloyd_max(d, bits)
        co, _, _, _ = codebook.lloyd_max_fd(d, bits)
        assert np.max(np.abs(c - co)) <= 1e-6 * np.max(np.abs(co))
        _cb_cache[key] = Codebooks(c, th)
    return _cb_cache[key]


def index_mismatches(gpu_idx: np.ndarray, ora_idx: np.ndarray, u: np.ndarray, th: np.ndarray):
    """(total mismatches, in-band, out-of-band): a mismatch is in band if the
    oracle's u lies within BAND * |theta| of a threshold between the two choices."""
    mis = np.nonzero(gpu_idx != ora_idx)
    n = len(mis[0])
    if n == 0:
        return 0, 0, 0
    g = gpu_idx[mis]
    o = ora_idx[mis]
    uu = u[mis]
    inband = 0
    for gi, oi, ui in zip(g, o, uu):
        lo, hi = min(gi, oi), max(gi, oi)
        # thresholds separating the two choices: theta_lo .. theta_{hi-1}
        ths = th[lo:hi]
        if hi - lo == 1 and abs(ui - ths[0]) <= BAND * abs(ths[0]):
            inband += 1
    return n, inband, n - inband


def tile_rel_max(y, ref, rows, tile: int = 256):
    """Largest relative Frobenius error over the kernel's 256 x 256 output tiles
    (restricted to the checked rows), so that one wrong tile cannot hide in the
    total."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rb = np.asarray(rows) // tile
    worst = 0.0
    for b in np.unique(rb):
        sel = rb == b
        for c0 in range(0, ref.shape[1], tile):
            r = ref[sel, c0:c0 + tile]
            den = np.linalg.norm(r)
            num = np.linalg.norm(y[sel, c0:c0 + tile] - r)
            if den > 0:
                worst = max(worst, float(num / den))
            elif num > 0:
                worst = float("inf")
    return worst


def rel_frob(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def to_device(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)       # exact: values are already bf16-representable
    return t.cuda()


def rotation(d: int, h: int, seed: int = 0, kind: str = "rpbh"):
    """Library rotation tables (checked bit-identical to the oracle's), host and device.
    kind: "rpbh" or "block_rht" (the ablation variant without the permutation)."""
    import torch
    if kind == "rpbh":
        perm, sign = oq.oq_build_rpbh(d, h, seed)
        po, so = rpbh.build_rpbh(d, h, seed)
    else:
        perm, sign = oq.oq_build_block_rht(d, h, seed)
        po, so = rpbh.build_block_rht(d, h, seed)
    assert np.array_equal(perm, po) and np.array_equal(sign, so)
    return perm, sign, torch.from_numpy(perm).cuda(), torch.from_numpy(sign).cuda()


CHUNK = 2048   # oracle rows per pass (bounds host memory at the full workload sizes)


def _chunks(rows, n=CHUNK):
    for i in range(0, len(rows), n):
        yield rows[i:i + n]


def check_activations(x: np.ndarray, dtype: str, h: int, bits: int, seed: int = 0, rows: Optional[np.ndarray] = None,
                      want_x_rot: bool = True, name: str = "", kind: str = "rpbh", keep_oracle: bool = False):
    """rotate-quantize x on the GPU; compare rows (all if None) with the oracle,
    in chunks of rows.  keep_oracle: the report also carries the oracle's own
    indices and norms of the checked rows ("_ia", "_s"), for the all-oracle product.

    Returns (x_idx device tensor, s device tensor, report dict)."""
    T, d = x.shape
    perm, sign, pd, sd = rotation(d, h, seed, kind)
    cb = library_codebook(d, bits)
    xd = to_device(x, dtype)
    x_idx, s, x_rot = oq.oq_rotate_quantize_act(xd, h, pd, sd, cb.th, bits, want_x_rot=want_x_rot)
    import torch
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else np.asarray(rows)
    xi_h = x_idx.cpu().numpy()
    s_h = s.cpu().numpy()
    xr_h = x_rot.cpu().numpy() if want_x_rot else None
    n = nin = nout = 0
    s_rel = xr_rel = 0.0
    keep_ia, keep_s = [], []
    for rc in _chunks(rows):
        xs = xd[torch.from_numpy(rc).long().cuda()].float().cpu().numpy().astype(np.float64)
        ia, s_o, xr_o, u_o = quant.quantize_activations(xs, perm, sign, h, cb.th)
        gi = quant.unpack(xi_h[rc], bits, d)
        m = index_mismatches(gi, ia, u_o, cb.th)
        n, nin, nout = n + m[0], nin + m[1], nout + m[2]
        s_rel = max(s_rel, float(np.max(np.abs(s_h[rc].astype(np.float64) - s_o) / np.maximum(s_o, 1e-30))))
        if want_x_rot:
            num = np.linalg.norm(xr_h[rc].astype(np.float64) - xr_o, axis=1)
            den = np.maximum(np.linalg.norm(xr_o, axis=1), 1e-30)
            xr_rel = max(xr_rel, float(np.max(num / den)))
        if keep_oracle:
            keep_ia.append(ia.astype(np.uint8))
            keep_s.append(s_o)
        del ia, s_o, xr_o, u_o, xs
    rep = {"name": name, "T": T, "d": d, "h": h, "bits": bits, "checked_rows": len(rows),
           "idx_mismatch": n, "idx_in_band": nin, "idx_out_of_band": nout, "s_rel": s_rel}
    if want_x_rot:
        rep["x_rot_rel"] = xr_rel
    log(f"[act] {rep}")
    if keep_oracle:
        rep["_ia"] = np.concatenate(keep_ia)
        rep["_s"] = np.concatenate(keep_s)
        rep["_rows"] = rows
    return x_idx, s, rep


def check_weights(W: np.ndarray, h: int, bits: int, seed: int = 0, name: str = "", kind: str = "rpbh"):
    """Quantize W on the GPU (fp64 path); indices must be bit-exact.  The
    report carries the oracle's indices and norms ("_iw", "_n")."""
    d_out, d = W.shape
    perm, sign, pd, sd = rotation(d, h, seed, kind)
    cb = library_codebook(d, bits)
    Wd = to_device(W, "f32")
    w_idx, w_norm = oq.oq_quantize_weights(Wd, h, pd, sd, cb.th, bits)
    iw, n_o, _, uw = quant.quantize_weights(W.astype(np.float64), perm, sign, h, cb.th)
    gi = quant.unpack(w_idx.cpu().numpy(), bits, d)
    n, nin, nout = index_mismatches(gi, iw, uw, cb.th)
    nrel = float(np.max(np.abs(w_norm.cpu().numpy() - n_o) / n_o))
    rep = {"name": name, "d_out": d_out, "d": d, "bits": bits, "idx_mismatch": n, "w_norm_rel": nrel}
    log(f"[w] {rep}")
    rep["_iw"] = iw.astype(np.uint8)
    rep["_n"] = n_o
    return w_idx, w_norm, rep


def run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca, cw, bias=None, epilogue=0, split=False, out_dtype=None,
             workspace=None):
    """One GEMM launch: oq_qlinear (whole tiles), or oq_qlinear_splitk with a
    zero-filled workspace of the size the library asks for (or the one given)."""
    if not split:
        return oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, ca, bits_a, cw, bits_w, bias=bias, epilogue=epilogue,
                             out_dtype=out_dtype)
    if workspace is None:
        workspace = oq.qlinear_workspace(s.shape[0], w_norm.shape[0], d, bits_a, bits_w)
    return oq.oq_qlinear_splitk(x_idx, s, w_idx, w_norm, d, ca, bits_a, cw, bits_w, workspace, bias=bias,
                                epilogue=epilogue, out_dtype=out_dtype)


def check_gemm(x_idx, s, w_idx, w_norm, d: int, bits_a: int, bits_w: int, bias=None, gelu=False,
               rows: Optional[np.ndarray] = None, name: str = "", out_dtype=None, split=False, workspace=None,
               all_oracle=None):
    """GEMM on the GPU vs the oracle's dequantized product of the GPU's own
    indices, s and norms (rows: all if None), in chunks of rows.

    split=True runs oq_qlinear_splitk (stream-K tail through a workspace).
    all_oracle = (act report, weight report) with the oracle's own indices:
    the error against the all-oracle product is reported too (information).
    With out_dtype=torch.bfloat16 the GEMM also runs with bf16 output; that
    tensor must hold the fp32 output rounded to nearest even, bit for bit
    (report key "bf16_equal"), and it is the one returned."""
    import torch
    ca = library_codebook(d, bits_a)
    cw = library_codebook(d, bits_w)
    bd = None if bias is None else torch.from_numpy(np.asarray(bias, dtype=np.float32)).cuda()
    epi = oq.OQ_EPI_GELU_ERF if gelu else oq.OQ_EPI_NONE
    y = run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bd, epilogue=epi, split=split,
                 workspace=workspace)
    torch.cuda.synchronize()
    T = s.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    iw = quant.unpack(w_idx.cpu().numpy(), bits_w, d)
    nw = w_norm.cpu().numpy()
    xi_h = x_idx.cpu().numpy()
    s_h = s.cpu().numpy()
    bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)
    num2 = den2 = 0.0
    tiles = {}
    finite = True
    a_num2 = a_den2 = 0.0
    if all_oracle is not None:
        ra, rw = all_oracle
        pos = {int(r): i for i, r in enumerate(ra["_rows"])}
    for rc in _chunks(rows):
        ia = quant.unpack(xi_h[rc], bits_a, d)
        ref = quant.dequantized_product(ia, s_h[rc], iw, nw, ca.c, cw.c, bias=bias_h, gelu=gelu)
        yg = y[torch.from_numpy(rc).long().cuda()].float().cpu().numpy().astype(np.float64)
        finite &= bool(np.all(np.isfinite(yg)))
        diff2 = (yg - ref) ** 2
        num2 += float(diff2.sum())
        den2 += float((ref ** 2).sum())
        rb = rc // 256
        for b in np.unique(rb):
            sel = rb == b
            for c0 in range(0, ref.shape[1], 256):
                key = (int(b), c0)
                t = tiles.setdefault(key, [0.0, 0.0])
                t[0] += float(diff2[sel, c0:c0 + 256].sum())
                t[1] += float((ref[sel, c0:c0 + 256] ** 2).sum())
        if all_oracle is not None:
            idx = np.array([pos[int(r)] for r in rc])
            ref_o = quant.dequantized_product(ra["_ia"][idx], ra["_s"][idx], rw["_iw"], rw["_n"], ca.c, cw.c,
                                              bias=bias_h, gelu=gelu)
            a_num2 += float(((yg - ref_o) ** 2).sum())
            a_den2 += float((ref_o ** 2).sum())
        del ia, ref, yg, diff2
    worst = 0.0
    for n2, d2 in tiles.values():
        if d2 > 0:
            worst = max(worst, float(np.sqrt(n2 / d2)))
        elif n2 > 0:
            worst = float("inf")
    err = float(np.sqrt(num2 / max(den2, 1e-300)))
    rep = {"name": name, "split": split, "T": T, "N": w_norm.shape[0], "K": d, "checked_rows": len(rows),
           "rel_frob": err, "tile_rel_max": worst, "finite": finite}
    if all_oracle is not None:
        rep["rel_frob_vs_all_oracle"] = float(np.sqrt(a_num2 / max(a_den2, 1e-300)))
    if out_dtype is not None:
        y16 = run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bd, epilogue=epi, split=split,
                       out_dtype=out_dtype, workspace=workspace)
        torch.cuda.synchronize()
        rep["bf16_equal"] = bool(torch.equal(y16.view(torch.int16), y.to(out_dtype).view(torch.int16)))
        y = y16
    log(f"[gemm] {rep}")
    return y, rep
