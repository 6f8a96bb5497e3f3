"""GPU parity of the INT4 round-to-nearest path (AdaLN modulation
projections) against the fp64 oracle, through the C ABI.

Bars: codes and scales bit-exact (both sides decide in fp64 with the same
fp32 scale); y within the fp32 summation bound of the oracle's fp64 product
of the same codes, scales and activations: per element
|y - y_ref| <= (d_in + 64) 2^-24 sum_k |s q x| + 2^-24 |bias|, and relative
Frobenius error <= 1e-5."""

import sys

import numpy as np
import pytest

from free_bit_quantization_amd import synth
from oracle import rtn

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _oq():
    from free_bit_quantization_amd import oq
    return oq


def _w_dev(W, dtype):
    t = torch.from_numpy(np.ascontiguousarray(W)).to("cuda:0")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def check_quantizer(W, group, w_dtype="f32"):
    oq = _oq()
    Wd = _w_dev(W, w_dtype)
    q, s = oq.oq_quantize_weights_int4(Wd, group)
    torch.cuda.synchronize()
    Wv = Wd.float().cpu().numpy()          # the values the kernel saw
    qo, so = rtn.quantize_int4_rtn(Wv, group)
    q_cpu, s_cpu = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(s_cpu.view(np.uint32), so.view(np.uint32)), "scales differ"
    po = rtn.pack_int4(qo)
    mism = int(np.count_nonzero(q_cpu != po))
    assert mism == 0, f"{mism} packed bytes differ"
    return q, s, qo, so


def check_linear(x, q, s, qo, so, group, bias=None, act="bf16"):
    oq = _oq()
    xt = torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    xt = xt.to(torch.bfloat16) if act == "bf16" else xt.to(torch.float16)
    bt = torch.from_numpy(bias).to("cuda:0") if bias is not None else None
    y = oq.oq_linear_w4a16(xt, q, s, group, bias=bt)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    xv = xt.float().cpu().numpy().astype(np.float64)
    yr = rtn.linear_w4a16(xv, qo, so, group, bias=bias)
    mag = np.abs(xv) @ np.abs(rtn.dequantize(qo, so, group)).T
    K = x.shape[1]
    bound = (K + 64) * U * mag + (U * np.abs(bias)[None, :] if bias is not None else 0.0) + 1e-30
    err = np.abs(yg - yr)
    assert np.all(np.isfinite(yg))
    worst = float(np.max(err / bound))
    frob = float(np.linalg.norm(yg - yr) / max(np.linalg.norm(yr), 1e-300))
    log(f"   max err / bound = {worst:.3g}, rel frob = {frob:.3g}")
    assert worst <= 1.0
    assert frob <= 1e-5
    return y


@pytest.mark.parametrize("d_out,d_in,group,w_dtype", [(300, 3072, 3072, "f32"), (300, 3072, 128, "bf16"),
                                                      (33, 256, 128, "f32"), (17, 1024, 256, "bf16")])
def test_int4_rtn_quantizer_bit_exact(d_out, d_in, group, w_dtype):
    log(f"== rtn quantizer {d_out}x{d_in} group {group} {w_dtype}")
    lin = synth.ModLinear("q", 1, d_in, d_out, group, w_outliers=max(1, d_in // 200))
    _, W = synth.gen_modulation(lin, seed=d_out, T=1)
    W[0, :] = 0.0                          # an all-zero row: s = 0, q = 0
    W[1, :] = 0.0
    W[1, 5] = -0.75                        # a single non-zero: -7 in its group
    check_quantizer(W, group, w_dtype)


@pytest.mark.parametrize("T,d_out,d_in,group,act,bias", [(2, 300, 3072, 3072, "bf16", False),
                                                         (1, 300, 3072, 128, "bf16", True),
                                                         (17, 45, 1024, 256, "f16", True),
                                                         (40, 129, 256, 128, "bf16", False),
                                                         (3, 16, 128, 128, "f16", False)])
def test_w4a16_linear_ragged(T, d_out, d_in, group, act, bias):
    log(f"== w4a16 T={T} {d_in}->{d_out} group {group} {act} bias={bias}")
    lin = synth.ModLinear("m", T, d_in, d_out, group, act_dtype=act, w_outliers=max(1, d_in // 200))
    x, W = synth.gen_modulation(lin, seed=T + d_out)
    q, s, qo, so = check_quantizer(W, group)
    b = synth.gen_bias(d_out, seed=T) if bias else None
    check_linear(x, q, s, qo, so, group, bias=b, act=act)


@pytest.mark.parametrize("k", [0, 1])
def test_full_flux_modulation_shape(k):
    lin = synth.modulation_workloads()["flux_adaln_mod_w4a16_b2"][k]
    log(f"== w4a16 full {lin.name}: T={lin.T} {lin.d_in}->{lin.d_out} group {lin.group}")
    x, W = synth.gen_modulation(lin, seed=k)
    q, s, qo, so = check_quantizer(W, lin.group)
    y1 = check_linear(x, q, s, qo, so, lin.group, bias=synth.gen_bias(lin.d_out, seed=k))
    # fixed-order reduction: a second call is bit-identical
    oq = _oq()
    xt = torch.from_numpy(x).to("cuda:0").to(torch.bfloat16)
    y2 = oq.oq_linear_w4a16(xt, q, s, lin.group, bias=torch.from_numpy(synth.gen_bias(lin.d_out, seed=k)).to("cuda:0"))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
