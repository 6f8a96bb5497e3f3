"""oq_qlinear_splitk_noalloc: the split codebook GEMM through the library's
fixed device scratch, for callers that cannot allocate.  Its output must
equal oq_qlinear_splitk's (same kernel, same split, own workspace) bit for
bit, and be within the GEMM bound of the fp64 oracle, on two calls in a row
where the second has the smaller input (the scratch keeps the first call's
contents)."""

import numpy as np
import pytest

import _parity as P
from free_bit_quantization_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(T, d, n, bits_w, bits_a, seed):
    lin = synth.Linear(f"noalloc-{T}x{d}x{n}", T, d, n, 256, bits_w, bits_a, "student_t", "bf16", 10, 30.0, 0.5,
                       5, 10.0)
    x, Wm = synth.gen_linear(lin, seed, 0)
    x_idx, s, ra = P.check_activations(x, "bf16", 256, bits_a, rows=np.arange(4), want_x_rot=False, name=lin.name)
    assert ra["idx_out_of_band"] == 0, ra
    w_idx, w_norm, rw = P.check_weights(Wm, 256, bits_w, name=lin.name)
    assert rw["idx_mismatch"] == 0, rw
    return lin, x_idx, s, w_idx, w_norm


@pytest.mark.parametrize("first,second", [((1024, 3072, 3072, 4, 8), (512, 3072, 1024, 4, 4)),
                                          ((2048, 3072, 9216, 4, 4), (2100, 3072, 300, 4, 4))])
def test_noalloc_matches_workspace_entry_point_twice(first, second):
    from free_bit_quantization_amd import oq
    for k, (T, d, n, bw, ba) in enumerate((first, second)):
        lin, x_idx, s, w_idx, w_norm = _case(T, d, n, bw, ba, seed=11 + k)
        assert oq.oq_qlinear_workspace_size(T, n, d, ba, bw) > 0, "the shape is expected to take the split"
        ca = P.library_codebook(d, ba).c
        cw = P.library_codebook(d, bw).c
        bias = torch.from_numpy(synth.gen_bias(n, k)).cuda()
        gelu = k == 1
        epi = oq.OQ_EPI_GELU_ERF if gelu else oq.OQ_EPI_NONE
        P.log(f"[noalloc] call {k}: T={T} d_in={d} d_out={n} W{bw}A{ba}")
        y_na = oq.oq_qlinear_splitk_noalloc(x_idx, s, w_idx, w_norm, d, ca, ba, cw, bw, bias=bias, epilogue=epi)
        ws = oq.qlinear_workspace(T, n, d, ba, bw)
        y_ws = oq.oq_qlinear_splitk(x_idx, s, w_idx, w_norm, d, ca, ba, cw, bw, ws, bias=bias, epilogue=epi)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"call {k}: differs from oq_qlinear_splitk"
        # and the bar of the parity tests against the oracle, on the rows of the split tiles
        rows = np.arange(max(0, T - 512), T)
        _, rg = P.check_gemm(x_idx, s, w_idx, w_norm, d, ba, bw, bias=bias.cpu().numpy(), gelu=gelu, rows=rows,
                             name=f"noalloc call {k}", split=True, workspace=ws)
        ia = P.quant.unpack(x_idx.cpu().numpy()[rows], ba, d)
        iw = P.quant.unpack(w_idx.cpu().numpy(), bw, d)
        ref = P.quant.dequantized_product(ia, s.cpu().numpy()[rows], iw, w_norm.cpu().numpy(), ca, cw,
                                          bias=bias.cpu().numpy(), gelu=gelu)
        err = P.rel_frob(y_na.cpu().numpy()[rows], ref)
        assert np.all(np.isfinite(y_na.cpu().numpy())) and err <= P.REL_GEMM, err
        del ws
