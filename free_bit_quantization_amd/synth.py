"""Seeded synthetic workloads for the quantized linear layer.

Holds the workload shapes and the input generators only: no step of the
quantization method is computed here, so both the HIP path and the fp64
oracle can take their inputs from this module.

The shapes stand in for DiT linears of the image and video models the
OrbitQuant pages evaluate (FLUX.1 double-stream blocks at 1024x1024, a
Wan 2.1 video FFN); trained weights and activations are not available, so
every tensor is drawn from a seeded distribution with the structure those
layers show (heavy-tailed activations with a few outlier channels and a
per-token scale, Xavier-scaled weights with a few outlier input columns).

Generator: ``numpy.random.default_rng`` on ``SeedSequence(seed)``; each
linear spawns five child streams in this order: activation values,
activation outlier channels, token scales, weight values, weight outlier
columns.  bf16 activations are rounded to nearest-even from fp32.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    T: int                 # tokens
    d_in: int              # K
    d_out: int             # N
    h: int                 # RPBH block size
    bits_w: int
    bits_a: int
    act: str               # "gauss" | "student_t"
    act_dtype: str         # "f32" | "bf16"
    act_outliers: int      # number of outlier channels
    act_outlier_scale: float
    token_lognormal: float  # sigma of the per-token LogNormal scale (0: none)
    w_outliers: int
    w_outlier_scale: float
    epilogue: str = "none"  # "none" | "gelu"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    linears: List[Linear]
    chained: bool = False   # MLP pair: the down input is GELU of the up output
    note: str = ""


def _lin(name, T, k, n, h, bw, ba, act="student_t", dtype="bf16", ao=None, aos=30.0,
         tok=0.5, wo=None, wos=10.0, epi="none"):
    if ao is None:
        ao = round(0.01 * k)
    if wo is None:
        wo = round(0.005 * k)
    return Linear(name, T, k, n, h, bw, ba, act, dtype, ao, aos, tok, wo, wos, epi)


def workloads() -> dict:
    """The workloads, by name."""
    w = {}
    w["single_w4a4_64x256x256"] = Workload(
        "single_w4a4_64x256x256",
        [Linear("single", 64, 256, 256, 64, 4, 4, "gauss", "f32", 4, 50.0, 0.0, 0, 1.0)],
        note="single linear, fp32 N(0,1) activations with 4 channels x50, h=64")
    w["flux_qkv_w4a4"] = Workload(
        "flux_qkv_w4a4",
        [_lin("qkv", 4608, 3072, 9216, 256, 4, 4)],
        note="FLUX.1-like double-stream QKV, 4096 image + 512 text tokens")
    w["flux_mlp_w2a4"] = Workload(
        "flux_mlp_w2a4",
        [_lin("up", 4608, 3072, 12288, 256, 2, 4, epi="gelu"),
         _lin("down", 4608, 12288, 3072, 256, 2, 4, dtype="f32")],
        chained=True,
        note="FLUX.1-like MLP pair; the down input is GELU(up output) in fp32")
    w["wan_ffn_w4a4"] = Workload(
        "wan_ffn_w4a4",
        [_lin("ffn", 32760, 5120, 13824, 256, 4, 4, ao=round(0.01 * 5120), aos=40.0, tok=0.0, wo=0)],
        note="Wan 2.1-like video FFN, 21x30x52 latent patches")
    lins = []
    for stream, T in (("img", 8192), ("txt", 1024)):
        lins += [_lin(f"{stream}_qkv", T, 3072, 9216, 256, 4, 8),
                 _lin(f"{stream}_out", T, 3072, 3072, 256, 4, 8),
                 _lin(f"{stream}_up", T, 3072, 12288, 256, 4, 8),
                 _lin(f"{stream}_down", T, 12288, 3072, 256, 4, 8)]
    w["flux_block_w4a8_b2"] = Workload(
        "flux_block_w4a8_b2", lins,
        note="all quantized linears of one FLUX.1-like double-stream block, batch 2 "
             "(cond + uncond concatenated along tokens); independent inputs per linear")
    w["flux_qkv_other_widths"] = Workload(
        "flux_qkv_other_widths",
        [_lin("qkv_w3a4", 4608, 3072, 9216, 256, 3, 4),
         _lin("qkv_w2a3", 4608, 3072, 9216, 256, 2, 3),
         _lin("qkv_w6a6", 4608, 3072, 9216, 256, 6, 6)],
        note="the FLUX.1-like QKV linear at the other index widths the pages name (W3A4, W2A3, W6A6)")
    return w


WORKLOAD_ORDER = ["single_w4a4_64x256x256", "flux_qkv_w4a4", "flux_mlp_w2a4",
                  "wan_ffn_w4a4", "flux_block_w4a8_b2", "flux_qkv_other_widths"]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); return fp32 holding it."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, index: int):
    ss = np.random.SeedSequence([seed, index])
    return [np.random.default_rng(s) for s in ss.spawn(5)]


def gen_linear(lin: Linear, seed: int = 0, index: int = 0, T: Optional[int] = None,
               need_act: bool = True):
    """Draw (x[T, d_in] fp32 holding bf16 or fp32 values, W[d_out, d_in] fp32).

    ``T`` overrides the token count (parity tests take a prefix workload of
    the same distribution); ``index`` selects the linear inside a workload.
    """
    T = lin.T if T is None else T
    r_act, r_ach, r_tok, r_w, r_wcol = _streams(seed, index)
    x = None
    if need_act:
        if lin.act == "gauss":
            x = r_act.standard_normal((T, lin.d_in), dtype=np.float32)
        else:
            x = r_act.standard_t(3.0, size=(T, lin.d_in)).astype(np.float32)
        if lin.act_outliers:
            ch = r_ach.choice(lin.d_in, lin.act_outliers, replace=False)
            x[:, ch] *= np.float32(lin.act_outlier_scale)
        if lin.token_lognormal > 0:
            g = np.exp(lin.token_lognormal * r_tok.standard_normal(T)).astype(np.float32)
            x *= g[:, None]
        if lin.act_dtype == "bf16":
            x = bf16_round(x)
    W = r_w.standard_normal((lin.d_out, lin.d_in), dtype=np.float32) * np.float32(1.0 / np.sqrt(lin.d_in))
    if lin.w_outliers:
        col = r_wcol.choice(lin.d_in, lin.w_outliers, replace=False)
        W[:, col] *= np.float32(lin.w_outlier_scale)
    return x, W


def gen_bias(n: int, seed: int = 0) -> np.ndarray:
    """A small seeded bias vector (tests of the bias epilogue)."""
    return (0.1 * np.random.default_rng(np.random.SeedSequence([seed, 999])).standard_normal(n)).astype(np.float32)


# ---- AdaLN modulation projections (INT4 round-to-nearest weights, 16-bit input)


@dataclasses.dataclass(frozen=True)
class ModLinear:
    """A modulation projection: the conditioning vector (one row per image of
    the batch) -> shift / scale / gate of the block's norms."""
    name: str
    T: int                  # rows (images in the batch)
    d_in: int
    d_out: int
    group: int              # input columns per INT4 scale (d_in = per output row)
    act_dtype: str = "bf16"  # "bf16" | "f16"
    w_outliers: int = 0
    w_outlier_scale: float = 10.0


def modulation_workloads() -> dict:
    """FLUX.1-like double-stream block, batch 2: two modulation projections
    of 3072 -> 6 x 3072 (image and text stream), per-row and per-128 scales."""
    return {
        "flux_adaln_mod_w4a16_b2": [ModLinear("img_mod", 2, 3072, 18432, 3072, w_outliers=15),
                                    ModLinear("txt_mod_g128", 2, 3072, 18432, 128, w_outliers=15)],
    }


def gen_modulation(lin: ModLinear, seed: int = 0, T: Optional[int] = None):
    """Draw (x[T, d_in] fp32 holding bf16 / fp16 values, W[d_out, d_in] fp32).

    x is SiLU of a standard normal conditioning vector (the modulation input
    is SiLU of the timestep + pooled-text embedding), rounded to the 16-bit
    type; W is N(0, 1/d_in) with a few outlier input columns."""
    T = lin.T if T is None else T
    r_act, r_w, r_wcol = [np.random.default_rng(s) for s in np.random.SeedSequence([seed, 7001]).spawn(3)]
    z = r_act.standard_normal((T, lin.d_in))
    x = (z / (1.0 + np.exp(-z))).astype(np.float32)
    if lin.act_dtype == "bf16":
        x = bf16_round(x)
    else:
        x = x.astype(np.float16).astype(np.float32)
    W = r_w.standard_normal((lin.d_out, lin.d_in), dtype=np.float32) * np.float32(1.0 / np.sqrt(lin.d_in))
    if lin.w_outliers:
        col = r_wcol.choice(lin.d_in, lin.w_outliers, replace=False)
        W[:, col] *= np.float32(lin.w_outlier_scale)
    return x, W
