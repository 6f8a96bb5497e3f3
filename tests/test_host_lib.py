"""liboq on the host: it loads, exports every symbol of include/oq.h, its
host calls agree with the oracle, and invalid arguments are rejected before
anything is launched (no device compute here)."""

import ctypes
import os
import re

import numpy as np
import pytest

from free_bit_quantization_amd import oq
from oracle import codebook, rpbh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "oq.h")).read()
    declared = set(re.findall(r"^\s*(?:const char\*|oq_status)\s+(oq_\w+)\s*\(", hdr, re.M))
    assert declared == set(oq.EXPORTS)
    L = oq.lib()
    for name in declared:
        assert hasattr(L, name)
    assert oq.oq_version().startswith("liboq")


@pytest.mark.parametrize("d,h,seed", [(8, 2, 0), (256, 64, 0), (3072, 256, 0), (5120, 256, 0), (12288, 256, 0), (96, 32, 77)])
def test_rpbh_bit_identical_to_oracle(d, h, seed):
    p, s = oq.oq_build_rpbh(d, h, seed)
    po, so = rpbh.build_rpbh(d, h, seed)
    np.testing.assert_array_equal(p, po)
    np.testing.assert_array_equal(s, so)


@pytest.mark.parametrize("d,h,seed", [(8, 2, 0), (256, 64, 0), (3072, 256, 0), (5120, 256, 0), (12288, 256, 0), (96, 32, 77)])
def test_block_rht_bit_identical_to_oracle(d, h, seed):
    p, s = oq.oq_build_block_rht(d, h, seed)
    po, so = rpbh.build_block_rht(d, h, seed)
    np.testing.assert_array_equal(p, po)
    np.testing.assert_array_equal(s, so)


@pytest.mark.parametrize("d,bits", [(3, 2), (256, 1), (256, 4), (3072, 2), (3072, 4), (3072, 8), (5120, 4),
                                    (12288, 2), (12288, 4), (12288, 8)])
def test_lloyd_max_agrees_with_oracle(d, bits):
    c, th, mse = oq.oq_lloyd_max(d, bits)
    co, tho, mseo, _ = codebook.lloyd_max_fd(d, bits)
    assert np.max(np.abs(c - co)) <= 1e-9 * np.max(np.abs(co))
    np.testing.assert_array_equal(th, 0.5 * (c[:-1] + c[1:]))
    assert abs(mse - mseo) <= 1e-8 * mseo
    # the library's codebook satisfies the oracle's fixed-point conditions
    m, _ = codebook.conditional_means(c, codebook.SphereMarginal(d))
    assert np.max(np.abs(c - m)) <= 1e-10 * np.max(np.abs(c))


def test_host_argument_errors():
    L = oq.lib()
    perm = np.zeros(8, np.int32)
    sign = np.zeros(8, np.int8)
    assert L.oq_build_rpbh(8, 3, 0, perm.ctypes.data, sign.ctypes.data) == oq.OQ_EINVAL
    assert L.oq_build_rpbh(8, 16, 0, perm.ctypes.data, sign.ctypes.data) == oq.OQ_EINVAL
    assert L.oq_build_rpbh(8, 2, 0, None, sign.ctypes.data) == oq.OQ_EINVAL
    assert L.oq_build_block_rht(8, 3, 0, perm.ctypes.data, sign.ctypes.data) == oq.OQ_EINVAL
    assert L.oq_build_block_rht(8, 16, 0, perm.ctypes.data, sign.ctypes.data) == oq.OQ_EINVAL
    assert L.oq_build_block_rht(8, 2, 0, perm.ctypes.data, None) == oq.OQ_EINVAL
    assert b"NULL" in L.oq_last_error()
    c = np.zeros(16)
    t = np.zeros(15)
    assert L.oq_lloyd_max(2, 4, c.ctypes.data, t.ctypes.data, None) == oq.OQ_EINVAL
    assert L.oq_lloyd_max(256, 9, c.ctypes.data, t.ctypes.data, None) == oq.OQ_EINVAL
    assert L.oq_lloyd_max(256, 4, c.ctypes.data, t.ctypes.data, None) == oq.OQ_OK
    assert L.oq_last_error() == b""


def _fake(n=1 << 20):
    # never dereferenced: validation fails before any launch
    return ctypes.c_void_p(n)


def test_device_calls_reject_bad_arguments_without_launching():
    L = oq.lib()
    _, th, _ = oq.oq_lloyd_max(256, 4)
    thp = th.ctypes.data
    bad_th = th.copy()
    bad_th[3] = bad_th[2]
    f = _fake()
    # rotate-quantize
    args = dict(x=f, dt=oq.OQ_BF16, T=4, d=256, h=64, perm=f, sign=f, th=thp, bits=4, idx=f, s=f, xr=None, st=None)

    def rq(**kw):
        a = dict(args, **kw)
        return L.oq_rotate_quantize_act(a["x"], a["dt"], a["T"], a["d"], a["h"], a["perm"], a["sign"], a["th"],
                                        a["bits"], a["idx"], a["s"], a["xr"], a["st"])
    assert rq(h=48) == oq.OQ_EINVAL
    assert rq(h=512) == oq.OQ_EINVAL            # h does not divide d
    assert rq(d=250) == oq.OQ_EINVAL
    assert rq(bits=5) == oq.OQ_EINVAL
    assert rq(T=-1) == oq.OQ_EINVAL
    assert rq(dt=7) == oq.OQ_EINVAL
    assert rq(x=None) == oq.OQ_EINVAL
    assert rq(th=bad_th.ctypes.data) == oq.OQ_EINVAL
    assert rq(th=None) == oq.OQ_EINVAL
    assert rq(d=768, h=256) == oq.OQ_EUNSUPPORTED   # d/16 = 48: no kernel plan
    assert rq(x=_fake((1 << 20) + 4)) == oq.OQ_EINVAL   # 16-byte vector loads need alignment
    assert rq(idx=_fake((1 << 20) + 8)) == oq.OQ_EINVAL
    assert rq(T=0) == oq.OQ_OK                       # valid no-op
    # weights
    assert L.oq_quantize_weights(f, oq.OQ_F32, 4, 256, 64, f, f, thp, 5, f, f, None) == oq.OQ_EINVAL
    assert L.oq_quantize_weights(f, oq.OQ_F32, -1, 256, 64, f, f, thp, 4, f, f, None) == oq.OQ_EINVAL
    assert L.oq_quantize_weights(None, oq.OQ_F32, 4, 256, 64, f, f, thp, 4, f, f, None) == oq.OQ_EINVAL
    assert L.oq_quantize_weights(f, oq.OQ_F32, 0, 256, 64, f, f, thp, 4, f, f, None) == oq.OQ_OK
    # GEMM
    c, _, _ = oq.oq_lloyd_max(256, 4)
    c2, _, _ = oq.oq_lloyd_max(256, 2)
    cp, c2p = c.ctypes.data, c2.ctypes.data
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 5, None, 0, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 5, f, None) == oq.OQ_EINVAL
    # the bf16-output flag combines with either activation, nothing else does
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0x200, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, oq.OQ_EPI_OUT_BF16 | 2, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(f, f, 0, f, f, 8, 256, cp, 4, cp, 4, None, oq.OQ_EPI_OUT_BF16 | oq.OQ_EPI_GELU_ERF, f,
                        None) == oq.OQ_OK
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, None, 4, cp, 4, None, 0, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(None, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(f, f, 4, f, f, 8, 96, cp, 4, cp, 4, None, 0, f, None) == oq.OQ_EUNSUPPORTED
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, c2p, 2, cp, 4, None, 0, f, None) == oq.OQ_EUNSUPPORTED  # A2
    assert L.oq_qlinear(f, f, 0, f, f, 8, 256, cp, 4, c2p, 2, None, 0, f, None) == oq.OQ_OK
    g = _fake((1 << 20) + 4)
    assert L.oq_qlinear(g, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, None) == oq.OQ_EINVAL
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, g, 0, f, None) == oq.OQ_EINVAL   # bias
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, g, None) == oq.OQ_EINVAL   # y


def test_int4_rtn_entry_points_reject_invalid_arguments():
    # only rejected calls and no-ops: nothing here may reach a launch
    L = oq.lib()
    f = _fake()
    g = _fake((1 << 20) + 4)
    q4 = L.oq_quantize_weights_int4
    assert q4(f, oq.OQ_F16, 8, 256, 256, f, f, None) == oq.OQ_EINVAL        # weights: fp32 / bf16 only
    assert q4(f, oq.OQ_F32, 8, 256, 64, f, f, None) == oq.OQ_EINVAL          # group not a multiple of 128
    assert q4(f, oq.OQ_F32, 8, 384, 256, f, f, None) == oq.OQ_EINVAL         # group does not divide d_in
    assert q4(f, oq.OQ_F32, -1, 256, 256, f, f, None) == oq.OQ_EINVAL
    assert q4(None, oq.OQ_F32, 8, 256, 256, f, f, None) == oq.OQ_EINVAL
    assert q4(f, oq.OQ_F32, 0, 256, 128, f, f, None) == oq.OQ_OK             # no rows: no-op
    lw = L.oq_linear_w4a16
    assert lw(f, oq.OQ_F32, 2, f, f, 64, 256, 256, None, f, None) == oq.OQ_EINVAL    # A16 only
    assert lw(f, oq.OQ_BF16, 2, f, f, 64, 192, 192, None, f, None) == oq.OQ_EINVAL   # d_in % 128
    assert lw(f, oq.OQ_BF16, 2, f, f, 64, 512, 192, None, f, None) == oq.OQ_EINVAL   # group
    assert lw(f, oq.OQ_BF16, -1, f, f, 64, 256, 256, None, f, None) == oq.OQ_EINVAL
    assert lw(None, oq.OQ_BF16, 2, f, f, 64, 256, 256, None, f, None) == oq.OQ_EINVAL
    assert lw(g, oq.OQ_BF16, 2, f, f, 64, 256, 256, None, f, None) == oq.OQ_EINVAL   # x alignment
    assert lw(f, oq.OQ_BF16, 2, g, f, 64, 256, 256, None, f, None) == oq.OQ_EINVAL   # q alignment
    assert lw(f, oq.OQ_BF16, 2, f, f, 64, 256, 256, g, f, None) == oq.OQ_EINVAL     # bias alignment
    assert lw(f, oq.OQ_F16, 65535 * 16 + 1, f, f, 64, 256, 256, None, f, None) == oq.OQ_EUNSUPPORTED
    assert lw(f, oq.OQ_F16, 0, f, f, 64, 256, 256, None, f, None) == oq.OQ_OK       # T = 0: no-op
    assert lw(f, oq.OQ_BF16, 4, f, f, 0, 256, 128, None, f, None) == oq.OQ_OK       # d_out = 0: no-op
    assert oq.lib().oq_last_error() is not None


def test_split_gemm_entry_points_reject_invalid_arguments():
    # only rejected calls, queries that need no device and no-ops
    L = oq.lib()
    f = _fake()
    g = _fake((1 << 20) + 4)
    c, _, _ = oq.oq_lloyd_max(256, 4)
    cp = c.ctypes.data
    sk = L.oq_qlinear_splitk
    assert sk(f, f, 4, f, f, 8, 256, cp, 4, cp, 5, None, 0, f, f, 1 << 30, None) == oq.OQ_EINVAL   # bits_w
    assert sk(None, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, f, 1 << 30, None) == oq.OQ_EINVAL
    assert sk(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, g, f, 1 << 30, None) == oq.OQ_EINVAL    # y alignment
    assert sk(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, _fake((1 << 20) + 16), 1 << 30,
              None) == oq.OQ_EINVAL                                                                  # workspace alignment
    assert b"256-byte" in L.oq_last_error()
    assert sk(f, f, 4, f, f, 8, 96, cp, 4, cp, 4, None, 0, f, f, 1 << 30, None) == oq.OQ_EUNSUPPORTED
    assert sk(f, f, 0, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, None, 0, None) == oq.OQ_OK            # T = 0
    ws = L.oq_qlinear_workspace_size
    n = ctypes.c_size_t(123)
    assert ws(4, 8, 256, 4, 4, None) == oq.OQ_EINVAL
    assert ws(-1, 8, 256, 4, 4, ctypes.addressof(n)) == oq.OQ_EINVAL
    assert ws(4, 8, 256, 5, 4, ctypes.addressof(n)) == oq.OQ_EINVAL
    assert ws(4, 8, 256, 2, 4, ctypes.addressof(n)) == oq.OQ_EUNSUPPORTED     # A2: no kernel
    assert ws(4, 8, 96, 4, 4, ctypes.addressof(n)) == oq.OQ_EUNSUPPORTED      # d_in not a multiple of 128
    assert ws(0, 8, 256, 4, 4, ctypes.addressof(n)) == oq.OQ_OK and n.value == 0


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(_gpu_visible(), reason="needs a host without a visible GPU (the calls would launch)")
def test_device_calls_without_a_device_return_edevice():
    # valid arguments on a host with no HIP device: the call reaches the
    # runtime, which reports no device; nothing can launch
    L = oq.lib()
    f = _fake()
    c, th, _ = oq.oq_lloyd_max(256, 4)
    cp, thp = c.ctypes.data, th.ctypes.data
    assert L.oq_qlinear(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, None) == oq.OQ_EDEVICE
    assert L.oq_last_error()
    assert L.oq_qlinear_splitk(f, f, 4, f, f, 8, 256, cp, 4, cp, 4, None, 0, f, None, 0, None) == oq.OQ_EDEVICE
    n = ctypes.c_size_t(0)
    assert L.oq_qlinear_workspace_size(4608, 9216, 3072, 4, 4, ctypes.addressof(n)) == oq.OQ_EDEVICE
    assert L.oq_rotate_quantize_act(f, oq.OQ_BF16, 4, 256, 64, f, f, thp, 4, f, f, None, None) == oq.OQ_EDEVICE
    assert L.oq_quantize_weights(f, oq.OQ_F32, 4, 256, 64, f, f, thp, 4, f, f, None) == oq.OQ_EDEVICE


@pytest.mark.parametrize("d,bits,steps", [(3072, 8, 0), (3072, 8, 2), (256, 4, 0), (12288, 4, 0)])
def test_lloyd_max_reports_non_convergence(monkeypatch, d, bits, steps):
    # with the Newton steps capped, the Lloyd steps alone leave the fixed-point
    # residual above 1e-10: OQ_ENOCONV, outputs still written (and ordered)
    L = oq.lib()
    n = 1 << bits
    c = np.full(n, np.nan)
    t = np.full(n - 1, np.nan)
    monkeypatch.setenv("OQ_LLOYD_MAX_NEWTON_STEPS", str(steps))
    assert L.oq_lloyd_max(d, bits, c.ctypes.data, t.ctypes.data, None) == oq.OQ_ENOCONV
    assert b"residual" in L.oq_last_error()
    assert np.all(np.isfinite(c)) and np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(t, 0.5 * (c[:-1] + c[1:]))
    monkeypatch.delenv("OQ_LLOYD_MAX_NEWTON_STEPS")
    assert L.oq_lloyd_max(d, bits, c.ctypes.data, t.ctypes.data, None) == oq.OQ_OK
    monkeypatch.setenv("OQ_LLOYD_MAX_NEWTON_STEPS", "garbage")   # not a count: the default cap
    assert L.oq_lloyd_max(d, bits, c.ctypes.data, t.ctypes.data, None) == oq.OQ_OK


def test_binding_checks_shapes_tables_and_devices_before_calling():
    # host tensors: every check that precedes the device check fires here,
    # and a well-shaped host tensor is refused as not being on the device
    torch = pytest.importorskip("torch")
    c, th, _ = oq.oq_lloyd_max(256, 4)
    T, d, n = 8, 256, 16
    x_idx = torch.zeros((T, d // 2), dtype=torch.uint8)
    s = torch.zeros(T)
    w_idx = torch.zeros((n, d // 2), dtype=torch.uint8)
    w_norm = torch.zeros(n)
    with pytest.raises(ValueError, match="centroids_a"):
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, c[:8], 4, c, 4)
    with pytest.raises(ValueError, match="centroids_w"):
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, c, 4, np.append(c, 0.0), 4)
    with pytest.raises(ValueError, match="x_idx"):
        oq.oq_qlinear(x_idx[:, :64], s, w_idx, w_norm, d, c, 4, c, 4)
    with pytest.raises(ValueError, match="w_idx"):
        oq.oq_qlinear(x_idx, s, w_idx[:-1], w_norm, d, c, 4, c, 4)
    with pytest.raises(ValueError, match="x_idx"):
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, 128, c, 4, c, 4)             # d_in disagrees with the indices
    with pytest.raises(ValueError, match="bias"):
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, c, 4, c, 4, bias=torch.zeros(n + 1))
    with pytest.raises(TypeError, match="s: expected torch.float32"):
        oq.oq_qlinear(x_idx, s.double(), w_idx, w_norm, d, c, 4, c, 4)
    with pytest.raises(TypeError, match="device"):
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, c, 4, c, 4)
    with pytest.raises(ValueError, match="thresholds"):
        oq.oq_rotate_quantize_act(torch.zeros((T, d)), 64, torch.zeros(d, dtype=torch.int32),
                                  torch.zeros(d, dtype=torch.int8), th[:-1], 4)
    with pytest.raises(ValueError, match="perm"):
        oq.oq_rotate_quantize_act(torch.zeros((T, d)), 64, torch.zeros(d - 1, dtype=torch.int32),
                                  torch.zeros(d, dtype=torch.int8), th, 4)
    with pytest.raises(ValueError, match="thresholds"):
        oq.oq_quantize_weights(torch.zeros((n, d)), 64, torch.zeros(d, dtype=torch.int32),
                               torch.zeros(d, dtype=torch.int8), np.append(th, 1.0), 4)
    with pytest.raises(ValueError, match="whole bytes"):
        oq.oq_rotate_quantize_act(torch.zeros((T, 250)), 2, torch.zeros(250, dtype=torch.int32),
                                  torch.zeros(250, dtype=torch.int8), oq.oq_lloyd_max(250, 3)[1], 3)


def test_fold_permutation_rejects_invalid_arguments():
    L = oq.lib()
    f = _fake()
    g = _fake((1 << 20) + 4)
    h = _fake(1 << 24)
    fo = L.oq_fold_permutation
    assert fo(f, f, None, 8, 256, 5, f, h, h, None, None) == oq.OQ_EINVAL          # bits_w
    assert fo(f, f, None, 8, 96, 2, f, h, h, None, None) == oq.OQ_EINVAL           # 24-byte rows
    assert fo(f, f, None, -1, 256, 4, f, h, h, None, None) == oq.OQ_EINVAL
    assert fo(None, f, None, 8, 256, 4, f, h, h, None, None) == oq.OQ_EINVAL
    assert fo(f, f, f, 8, 256, 4, f, h, h, None, None) == oq.OQ_EINVAL             # bias without bias_out
    assert fo(g, f, None, 8, 256, 4, f, h, h, None, None) == oq.OQ_EINVAL          # alignment
    assert fo(f, f, None, 8, 256, 4, f, _fake((1 << 20) + 256), h, None, None) == oq.OQ_EINVAL   # overlap
    assert b"overlap" in L.oq_last_error()
    assert fo(f, f, None, 0, 256, 4, f, h, h, None, None) == oq.OQ_OK              # no rows
