"""The MLP pair with the down projection's permutation folded into the up
projection (oq_fold_permutation), against the unfolded chain and the fp64
oracle.

Folded chain: rotate-quantize x, up GEMM with the folded rows and the GELU
epilogue -> h' (= h with its columns in the down rotation's permutation
order), rotate-quantize h' with the identity permutation and the down
rotation's signs, down GEMM.  Checks:
  * h' equals the unfolded chain's h with its columns permuted, bit for bit;
  * the down activation indices agree with the fp64 oracle's rotation of the
    unfolded h (band rule), and the norms within 1e-5;
  * the down GEMM within 2e-3 of the oracle's product of the GPU's own
    indices; the whole chain's error against the all-oracle chain is reported.
"""

import numpy as np
import pytest

import _parity as P
from free_bit_quantization_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.workloads()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _chain(T, hidden_dtype, act_rows, gemm_rows, split=False):
    from free_bit_quantization_amd import oq
    from oracle import quant
    up, down = W["flux_mlp_w2a4"].linears
    K, H, N, hb = up.d_in, up.d_out, down.d_out, up.h
    x, W_up = synth.gen_linear(up, 0, 0, T=T)
    _, W_dn = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    bias_up = synth.gen_bias(H, 3)
    P.log(f"== folded MLP chain T={T} hidden={hidden_dtype}")
    # up: activations and weights (unfolded), then the folded copies
    xi, s_up, ra = P.check_activations(x, "bf16", hb, up.bits_a, rows=act_rows, want_x_rot=False, name="up")
    assert ra["idx_out_of_band"] == 0, ra
    wi_up, wn_up, rw = P.check_weights(W_up, hb, up.bits_w, name="up")
    assert rw["idx_mismatch"] == 0, rw
    perm_d, sign_d, pd_d, sd_d = P.rotation(H, hb, 0)
    b_up = torch.from_numpy(bias_up).cuda()
    wi_f, wn_f, b_f = oq.oq_fold_permutation(wi_up, wn_up, pd_d, K, up.bits_w, bias=b_up)
    cb_a, cb_w = P.library_codebook(K, up.bits_a), P.library_codebook(K, up.bits_w)
    od = torch.bfloat16 if hidden_dtype == "bf16" else torch.float32

    def gemm(xi_, s_, wi_, wn_, d, ca, ba, cw, bw, bias=None, epi=0):
        return P.run_gemm(xi_, s_, wi_, wn_, d, ba, bw, ca, cw, bias=bias, epilogue=epi, split=split, out_dtype=od)

    h = gemm(xi, s_up, wi_up, wn_up, K, cb_a.c, up.bits_a, cb_w.c, up.bits_w, b_up, oq.OQ_EPI_GELU_ERF)
    hf = gemm(xi, s_up, wi_f, wn_f, K, cb_a.c, up.bits_a, cb_w.c, up.bits_w, b_f, oq.OQ_EPI_GELU_ERF)
    torch.cuda.synchronize()
    hp = h[:, torch.from_numpy(perm_d).long().cuda()]
    if not split:
        # each output element is the same dot product in the same order
        assert torch.equal(hf, hp), "folded up output is not h[:, perm]"
    else:
        # the split cuts a tile's K range by the tile's place in the launch, so
        # a permuted column can be summed in another order: fp32 rounding only
        d = (hf.float() - hp.float()).abs().max().item()
        tol = (2.0 ** -7 if od == torch.bfloat16 else 1e-5) * hp.float().abs().max().item()
        P.log(f"[fold up] split: max |h' - h[:, perm]| = {d:.3e} (bound {tol:.3e})")
        assert d <= tol
    # down rotate-quantize of h' with the identity permutation and the down signs
    ident = torch.arange(H, dtype=torch.int32, device="cuda")
    cb_da, cb_dw = P.library_codebook(H, down.bits_a), P.library_codebook(H, down.bits_w)
    xi_d, s_d, _ = oq.oq_rotate_quantize_act(hf, hb, ident, sd_d, cb_da.th, down.bits_a)
    torch.cuda.synchronize()
    # the oracle rotates the hidden state the GPU consumed, put back in the
    # unfolded order (column perm[i] of the unfolded h is column i of h'),
    # with the down rotation's own tables
    rows = np.arange(T) if act_rows is None else act_rows
    hf64 = hf.float().cpu().numpy().astype(np.float64)[rows]
    h64 = np.empty_like(hf64)
    h64[:, perm_d] = hf64
    ia, s_o, _, u_o = quant.quantize_activations(h64, perm_d, sign_d, hb, cb_da.th)
    gi = quant.unpack(xi_d.cpu().numpy()[rows], down.bits_a, H)
    n, nin, nout = P.index_mismatches(gi, ia, u_o, cb_da.th)
    s_rel = float(np.max(np.abs(s_d.cpu().numpy()[rows] - s_o) / np.maximum(s_o, 1e-30)))
    P.log(f"[fold act] rows={len(rows)} mismatches={n} in_band={nin} out_of_band={nout} s_rel={s_rel:.2e}")
    assert nout == 0 and s_rel <= P.REL_S
    # down GEMM on the folded chain's indices
    wi_d, wn_d, rw = P.check_weights(W_dn, hb, down.bits_w, name="down")
    assert rw["idx_mismatch"] == 0, rw
    y, rg = P.check_gemm(xi_d, s_d, wi_d, wn_d, H, down.bits_a, down.bits_w, rows=gemm_rows, name="down (folded)",
                         split=split)
    assert rg["finite"] and rg["rel_frob"] <= P.REL_GEMM and rg["tile_rel_max"] <= P.REL_GEMM, rg
    return x, W_up, bias_up, W_dn, y


def test_folded_mlp_chain_prefix_fp32_hidden():
    _chain(264, "f32", None, None)


def test_folded_mlp_chain_prefix_bf16_hidden_split():
    _chain(264, "bf16", None, None, split=True)


def test_folded_mlp_chain_full_size_against_the_all_oracle_chain():
    # the FLUX MLP shape, every token's down indices checked; the whole
    # chain's error against the all-oracle chain (fp64, unfolded, the oracle's
    # own indices everywhere) is reported and bounded loosely: it is the
    # fp16 table rounding of two GEMMs passed through GELU and a requantization
    from oracle import quant
    up, down = W["flux_mlp_w2a4"].linears
    T = up.T
    rows = P.sample_rows(T, 96)
    x, W_up, bias_up, W_dn, y = _chain(T, "f32", None, rows)
    perm_u, sign_u, _, _ = P.rotation(up.d_in, up.h, 0)
    perm_d, sign_d, _, _ = P.rotation(up.d_out, up.h, 0)
    cb = {(d, b): P.library_codebook(d, b) for d in (up.d_in, up.d_out) for b in (2, 4)}
    xs = x.astype(np.float64)[rows]
    ia, s_a, _, _ = quant.quantize_activations(xs, perm_u, sign_u, up.h, cb[(up.d_in, 4)].th)
    iw, n_w, _, _ = quant.quantize_weights(W_up.astype(np.float64), perm_u, sign_u, up.h, cb[(up.d_in, 2)].th)
    h = quant.dequantized_product(ia, s_a, iw, n_w, cb[(up.d_in, 4)].c, cb[(up.d_in, 2)].c, bias=bias_up, gelu=True)
    ia2, s2, _, _ = quant.quantize_activations(h, perm_d, sign_d, up.h, cb[(up.d_out, 4)].th)
    iw2, n2, _, _ = quant.quantize_weights(W_dn.astype(np.float64), perm_d, sign_d, up.h, cb[(up.d_out, 2)].th)
    y_o = quant.dequantized_product(ia2, s2, iw2, n2, cb[(up.d_out, 4)].c, cb[(up.d_out, 2)].c)
    err = P.rel_frob(y.cpu().numpy()[rows], y_o)
    P.log(f"[fold chain] GPU folded chain vs all-oracle unfolded chain: rel Frobenius {err:.3e} over {len(rows)} rows")
    assert err <= 2e-2, err
