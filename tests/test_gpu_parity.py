"""GPU parity: liboq's kernels against the fp64 oracle on the same seeded
inputs, through the C ABI (Python binding = marshalling only).

Bars: packed indices bit-exact except within 1e-11 |theta| of a threshold
(fp64 summation order; weights: bit-exact); rotated activations and norms within 1e-5 relative;
GEMM within 2e-3 relative Frobenius of the oracle's dequantized product of
the GPU's own indices, norms and scales."""

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


def _assert_act(rep):
    assert rep["idx_out_of_band"] == 0, rep
    assert rep["s_rel"] <= P.REL_S, rep
    if "x_rot_rel" in rep:
        assert rep["x_rot_rel"] <= P.REL_XROT, rep


def _assert_w(rep):
    assert rep["idx_mismatch"] == 0, rep
    assert rep["w_norm_rel"] <= 1e-6, rep


def _assert_gemm(rep):
    assert rep["finite"], rep
    assert rep["rel_frob"] <= P.REL_GEMM, rep
    assert rep["tile_rel_max"] <= P.REL_GEMM, rep


def run_linear(lin, index=0, T=None, seed=0, bias=False, act_rows=None, gemm_rows=None, x=None, W_=None,
               x_dtype=None, kind="rpbh", out_dtype=None, split=False):
    """One linear through the GPU path against the oracle: every checked
    activation row and GEMM row (all rows when act_rows / gemm_rows are None).
    The GEMM's error against the all-oracle product (the oracle's own indices,
    norms and scales) is reported as information when the GEMM rows are a
    subset of the checked activation rows."""
    P.log(f"== linear {lin.name} T={T or lin.T} K={lin.d_in} N={lin.d_out} W{lin.bits_w}A{lin.bits_a}")
    xg, Wg = synth.gen_linear(lin, seed, index, T=T, need_act=x is None)
    x = xg if x is None else x
    W_ = Wg if W_ is None else W_
    x_idx, s, ra = P.check_activations(x, x_dtype or lin.act_dtype, lin.h, lin.bits_a, rows=act_rows,
                                       want_x_rot=True, name=lin.name, kind=kind, keep_oracle=True)
    _assert_act(ra)
    w_idx, w_norm, rw = P.check_weights(W_, lin.h, lin.bits_w, name=lin.name, kind=kind)
    _assert_w(rw)
    b = synth.gen_bias(lin.d_out, seed) if bias else None
    rows_g = np.arange(x.shape[0]) if gemm_rows is None else np.asarray(gemm_rows)
    both = set(rows_g.tolist()) <= set(ra["_rows"].tolist())
    y, rg = P.check_gemm(x_idx, s, w_idx, w_norm, lin.d_in, lin.bits_a, lin.bits_w, bias=b,
                         gelu=lin.epilogue == "gelu", rows=gemm_rows, name=lin.name, out_dtype=out_dtype,
                         split=split, all_oracle=(ra, rw) if both else None)
    _assert_gemm(rg)
    if out_dtype is not None:
        assert rg["bf16_equal"], rg
    return y


# ---- small and prefix workloads (oracle over every output) ------------------


def test_single_linear_w4a4_full():
    run_linear(W["single_w4a4_64x256x256"].linears[0])


def test_single_linear_with_bias():
    run_linear(W["single_w4a4_64x256x256"].linears[0], bias=True, seed=3)


def test_flux_qkv_prefix_ragged():
    run_linear(W["flux_qkv_w4a4"].linears[0], T=300)


def test_flux_mlp_chain_prefix():
    up, down = W["flux_mlp_w2a4"].linears
    y_up = run_linear(up, index=0, T=264)
    # the down projection takes GELU(up) in fp32, exactly as the GPU produced it
    x_down = y_up.cpu().numpy().astype(np.float32)
    _, W_down = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    run_linear(down, index=1, T=264, x=x_down, W_=W_down, x_dtype="f32")


def test_flux_mlp_chain_prefix_bf16_hidden():
    # the hidden state kept in bf16: the up GEMM writes GELU(y) rounded to
    # bf16 and the down rotate-quantize reads that tensor as it is
    up, down = W["flux_mlp_w2a4"].linears
    h16 = run_linear(up, index=0, T=264, out_dtype=torch.bfloat16)
    x_down = h16.float().cpu().numpy()
    _, W_down = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    run_linear(down, index=1, T=264, x=x_down, W_=W_down, x_dtype="bf16")


def test_wan_ffn_prefix_ragged():
    run_linear(W["wan_ffn_w4a4"].linears[0], T=200)


@pytest.mark.parametrize("k", range(8))
def test_flux_block_w4a8_prefix(k):
    lin = W["flux_block_w4a8_b2"].linears[k]
    run_linear(lin, index=k, T=136 if lin.T > 1024 else 72)


# ---- rotation variant (ablation without the permutation): same kernels, other tables


def test_block_rht_tables_through_both_kernels():
    run_linear(W["flux_qkv_w4a4"].linears[0], T=200, kind="block_rht")
    run_linear(W["single_w4a4_64x256x256"].linears[0], kind="block_rht")


# ---- edge cases ----------------------------------------------------------------


@pytest.mark.parametrize("d,h,dtype", [(256, 2, "f32"), (256, 4, "bf16"), (256, 16, "f32"), (512, 32, "bf16"),
                                       (1024, 64, "f32"), (1024, 128, "bf16"), (2048, 256, "bf16"),
                                       (64, 64, "f32"), (16, 16, "bf16"), (12288, 256, "f32"),
                                       (4096, 256, "bf16"), (5120, 64, "bf16"), (5120, 256, "bf16"),
                                       (4096, 64, "f32")])
@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_rotate_quantize_shapes_and_widths(d, h, dtype, bits):
    rng = np.random.default_rng(d * 7 + h + bits)
    T = 37
    x = rng.standard_t(3, size=(T, d)).astype(np.float32) * np.float32(3.0)
    if dtype == "bf16":
        x = synth.bf16_round(x)
    _, _, rep = P.check_activations(x, dtype, h, bits, name=f"shape d={d} h={h}")
    _assert_act(rep)


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("d_out,d,h", [(40, 3072, 256), (17, 1024, 64), (9, 256, 16)])
def test_weight_quantization_non_byte_widths(bits, d_out, d, h):
    rng = np.random.default_rng(bits * 100 + d)
    Wm = rng.standard_normal((d_out, d)).astype(np.float32) / np.float32(np.sqrt(d))
    _, _, rep = P.check_weights(Wm, h, bits, name=f"w{bits} d={d}")
    _assert_w(rep)


def test_zero_rows_single_token_and_repeatability():
    rng = np.random.default_rng(5)
    d, h, bits = 3072, 256, 4
    x = synth.bf16_round(rng.standard_normal((5, d)).astype(np.float32))
    x[1] = 0.0
    x[3] = 0.0
    x_idx, s, rep = P.check_activations(x, "bf16", h, bits, name="zero rows")
    _assert_act(rep)
    s_h = s.cpu().numpy()
    assert s_h[1] == 0.0 and s_h[3] == 0.0
    idx = x_idx.cpu().numpy()
    # a zero row quantizes every coordinate to the index just below 0 (L/2 - 1)
    assert np.all(idx[1] == (7 | (7 << 4)))
    # one token
    _, _, rep1 = P.check_activations(x[:1], "bf16", h, bits, name="T=1")
    _assert_act(rep1)
    # repeat runs give bit-identical outputs
    xi2, s2, _ = P.check_activations(x, "bf16", h, bits, want_x_rot=False, name="repeat")
    assert np.array_equal(xi2.cpu().numpy(), idx) and np.array_equal(s2.cpu().numpy(), s_h)


def test_gemm_ragged_m_and_n_tails_and_bias():
    # T and d_out not multiples of the 256 x 256 tile
    rng = np.random.default_rng(9)
    d, h = 1024, 256
    lin = synth.Linear("ragged", 333, d, 300, h, 4, 4, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0)
    run_linear(lin, bias=True)
    del rng


def test_gemm_gelu_epilogue_w2a4():
    lin = synth.Linear("gelu", 130, 1024, 520, 256, 2, 4, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0, "gelu")
    run_linear(lin, bias=True)


@pytest.mark.parametrize("bits_w,bits_a,T,d,d_out,h", [(3, 4, 300, 1024, 520, 256), (2, 3, 130, 3072, 300, 256),
                                                      (6, 6, 200, 1024, 272, 64), (3, 4, 17, 256, 9, 16),
                                                      (6, 6, 1, 64, 3, 64)])
def test_gemm_non_byte_index_widths(bits_w, bits_a, T, d, d_out, h):
    # 3- and 6-bit indices (W3A4, W2A3, W6A6): expanded to 4/8 bits while staged
    lin = synth.Linear(f"w{bits_w}a{bits_a}", T, d, d_out, h, bits_w, bits_a, "student_t", "bf16", 10, 30.0, 0.5,
                       5, 10.0)
    run_linear(lin, bias=True, seed=bits_w * 10 + bits_a)


@pytest.mark.parametrize("bits_w,bits_a,T,d,d_out,h", [(2, 8, 300, 1024, 260, 256), (4, 4, 70, 1024, 258, 64),
                                                      (2, 4, 33, 512, 131, 32), (4, 8, 129, 3072, 517, 256)])
def test_gemm_byte_widths_ragged_columns(bits_w, bits_a, T, d, d_out, h):
    # W2A8 and d_out not a multiple of 4 (the per-element store path of the epilogue)
    lin = synth.Linear(f"w{bits_w}a{bits_a}r", T, d, d_out, h, bits_w, bits_a, "student_t", "bf16", 10, 30.0, 0.5,
                       5, 10.0)
    run_linear(lin, bias=True, seed=bits_w * 100 + d_out)


def test_gemm_repeatable():
    lin = W["single_w4a4_64x256x256"].linears[0]
    x, Wm = synth.gen_linear(lin, 0, 0)
    x_idx, s, _ = P.check_activations(x, "f32", lin.h, 4, want_x_rot=False)
    w_idx, w_norm, _ = P.check_weights(Wm, lin.h, 4)
    y1, _ = P.check_gemm(x_idx, s, w_idx, w_norm, lin.d_in, 4, 4)
    y2, _ = P.check_gemm(x_idx, s, w_idx, w_norm, lin.d_in, 4, 4)
    assert torch.equal(y1, y2)


# ---- stream-K: the last, partial round of tiles split by K stages -----------------


def _gemm_twice(lin, rows, seed, bias=False, gelu=False):
    """oq_qlinear_splitk on two scale vectors in a row through one workspace,
    every tile of both checked: the second launch must not consume the first
    one's partial tiles.  Then oq_qlinear (whole tiles) on the same inputs:
    the tiles that neither launch splits are bit-identical."""
    from free_bit_quantization_amd import oq
    x, Wm = synth.gen_linear(lin, seed, 0)
    x_idx, s, ra = P.check_activations(x, lin.act_dtype, lin.h, lin.bits_a, rows=np.arange(min(8, lin.T)),
                                       want_x_rot=False, name=lin.name)
    _assert_act(ra)
    w_idx, w_norm, rw = P.check_weights(Wm, lin.h, lin.bits_w, name=lin.name)
    _assert_w(rw)
    b = synth.gen_bias(lin.d_out, seed) if bias else None
    ws = oq.qlinear_workspace(lin.T, lin.d_out, lin.d_in, lin.bits_a, lin.bits_w)
    assert ws is not None, "the shape is expected to take the split"
    ys = []
    for k, scale in enumerate((1.0, 1.75)):
        sk = s * scale
        y, rg = P.check_gemm(x_idx, sk, w_idx, w_norm, lin.d_in, lin.bits_a, lin.bits_w, bias=b, gelu=gelu,
                             rows=rows, name=f"{lin.name}-launch{k}", split=True, workspace=ws)
        _assert_gemm(rg)
        ys.append(y)
    y_whole, rg = P.check_gemm(x_idx, s * 1.75, w_idx, w_norm, lin.d_in, lin.bits_a, lin.bits_w, bias=b, gelu=gelu,
                               rows=rows, name=f"{lin.name}-whole")
    _assert_gemm(rg)
    return ys[1], y_whole


def _untouched_tiles_equal(y_split, y_whole, T, N, n_dp):
    # tiles [0, n_dp) of the grouped raster order are computed the same way by
    # both entry points; compare the rows of every 256-row block whose tiles
    # all come before the split (the raster walks 4 block rows at a time)
    ntn = (N + 255) // 256
    full_groups = n_dp // (4 * ntn)
    r = min(T, full_groups * 4 * 256)
    assert torch.equal(y_split[:r], y_whole[:r])
    return r


@pytest.mark.parametrize("T,d,d_out,bits_w,bits_a", [(1024, 3072, 3072, 4, 8), (1024, 12288, 3072, 4, 8),
                                                     (2100, 3072, 300, 4, 4), (1000, 3072, 2000, 2, 4),
                                                     (512, 3072, 1024, 4, 4),    # 8 tiles: one per class, 4 pieces
                                                     (1024, 2048, 512, 4, 4),    # 16 K stages per tile
                                                     (1024, 1024, 1024, 6, 6)])  # 6-bit widths (128 x 64 blocks)
def test_stream_k_split_tiles(T, d, d_out, bits_w, bits_a):
    # fewer tiles than CUs (8 to 48, some ragged): every tile is split by K
    # stages over 2-5 workgroups (stream-K); bias and GELU on the ragged shape
    # (the finisher applies them after summing the partials)
    lin = synth.Linear(f"sk-{T}x{d}x{d_out}", T, d, d_out, 256, bits_w, bits_a, "student_t", "bf16", 10, 30.0,
                       0.5, 5, 10.0)
    ragged = d_out % 256 != 0
    _gemm_twice(lin, np.arange(T), seed=T + d, bias=ragged, gelu=ragged)


@pytest.mark.parametrize("T,d,d_out,bits_w,bits_a,rows0,n_dp", [
    (2048, 3072, 9216, 4, 4, 1024, 256),     # 288 tiles: one whole round, 32 tiles of 24 stages split
    (8192, 12288, 3072, 4, 8, 5120, 256)])   # 384 tiles: one whole round, 128 tiles of 192 stages split
def test_last_round_split_after_whole_rounds_twice(T, d, d_out, bits_w, bits_a, rows0, n_dp):
    # more tiles than CUs: the first round whole, the tail split by K stages;
    # the tail's rows (grouped raster order, 4 block rows at a time) checked
    # tile by tile on two launches in a row, the rows before it bit-identical
    # to the whole-tile entry point
    lin = synth.Linear(f"tail-{T}x{d}x{d_out}", T, d, d_out, 256, bits_w, bits_a, "student_t", "bf16", 10, 30.0,
                       0.5, 5, 10.0)
    y_split, y_whole = _gemm_twice(lin, np.arange(rows0, T), seed=5)
    assert _untouched_tiles_equal(y_split, y_whole, T, d_out, n_dp) == rows0


def test_split_workspace_size_and_rejection():
    from free_bit_quantization_amd import oq
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = oq.oq_qlinear_workspace_size(2048, 9216, 3072, 4, 4)              # 288 tiles: a tail of 32 split
    slots_off = 256 + ((4 * cus + 255) // 256) * 256
    assert n == slots_off + cus * 256 * 256 * 4, (n, cus)
    assert oq.oq_qlinear_workspace_size(4608, 9216, 3072, 4, 4) == 0     # a tail of 136 short tiles: whole
    assert oq.oq_qlinear_workspace_size(256, 256, 256, 4, 4) == 0        # 2 K stages: no split
    assert oq.oq_qlinear_workspace_size(256, 256, 3072, 4, 4) == n       # one tile of 24 stages: split
    lin = synth.Linear("ws", 512, 3072, 1024, 256, 4, 4, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0)
    x, Wm = synth.gen_linear(lin, 1, 0)
    x_idx, s, _ = P.check_activations(x, "bf16", 256, 4, rows=np.arange(4), want_x_rot=False)
    w_idx, w_norm, _ = P.check_weights(Wm, 256, 4)
    cb = P.library_codebook(3072, 4)
    need = oq.oq_qlinear_workspace_size(512, 1024, 3072, 4, 4)
    assert need > 0
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(oq.OQError) as e:
        oq.oq_qlinear_splitk(x_idx, s, w_idx, w_norm, 3072, cb.c, 4, cb.c, 4, small)
    assert e.value.status == oq.OQ_EINVAL and "workspace" in str(e.value)
    with pytest.raises(oq.OQError):
        oq.oq_qlinear_splitk(x_idx, s, w_idx, w_norm, 3072, cb.c, 4, cb.c, 4, None)
    # a shape without a split (2 K stages per tile) ignores the workspace
    g = torch.Generator(device="cuda").manual_seed(3)
    xi2 = torch.randint(0, 256, (300, 128), dtype=torch.uint8, device="cuda", generator=g)
    wi2 = torch.randint(0, 256, (300, 128), dtype=torch.uint8, device="cuda", generator=g)
    s2 = torch.rand(300, device="cuda", generator=g) + 0.5
    n2 = torch.rand(300, device="cuda", generator=g) + 0.5
    cb2 = P.library_codebook(256, 4)
    assert oq.oq_qlinear_workspace_size(300, 300, 256, 4, 4) == 0
    y = oq.oq_qlinear_splitk(xi2, s2, wi2, n2, 256, cb2.c, 4, cb2.c, 4, None)
    y0 = oq.oq_qlinear(xi2, s2, wi2, n2, 256, cb2.c, 4, cb2.c, 4)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_split_launch_generations_across_the_wrap():
    # The workspace header (one 64-bit word: generation, workgroups started)
    # set just below the 32-bit wrap: four split launches in a row go through
    # generations 0xFFFFFFFD, 0xFFFFFFFE, 0 and 1.  After each launch the
    # header must hold the next generation and a zero count, and y must equal
    # bit for bit the same launch on a fresh zero-filled workspace (the split's
    # summation order is fixed, so any stale or missed partial would show).
    from free_bit_quantization_amd import oq
    g = torch.Generator(device="cuda").manual_seed(11)
    T, K, N = 512, 3072, 1024                     # 8 tiles of 24 stages: every tile split
    x_idx = torch.randint(0, 256, (T, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    w_idx = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    s = torch.rand(T, device="cuda", generator=g) + 0.5
    wn = torch.rand(N, device="cuda", generator=g) + 0.5
    cb = P.library_codebook(K, 4)
    ws = oq.qlinear_workspace(T, N, K, 4, 4)
    assert ws is not None
    ws[:8].copy_(torch.tensor([0xFFFFFFFD, 0], dtype=torch.int64).to(torch.uint32).view(torch.uint8)[:8])

    def header():
        h = ws[:8].cpu().view(torch.int32).numpy().view(np.uint32)
        return int(h[0]), int(h[1])

    assert header() == (0xFFFFFFFD, 0)
    expect_gen = [0xFFFFFFFE, 0, 1, 2]
    for k, scale in enumerate((1.0, 1.5, 0.75, 2.0)):
        y = oq.oq_qlinear_splitk(x_idx, s * scale, w_idx, wn, K, cb.c, 4, cb.c, 4, ws)
        fresh = oq.qlinear_workspace(T, N, K, 4, 4)
        y_ref = oq.oq_qlinear_splitk(x_idx, s * scale, w_idx, wn, K, cb.c, 4, cb.c, 4, fresh)
        torch.cuda.synchronize()
        assert header() == (expect_gen[k], 0), (k, header())
        assert bool(torch.isfinite(y).all())
        assert torch.equal(y, y_ref), k


# ---- bf16 output: the fp32 result rounded to nearest even, bit for bit -----------


@pytest.mark.parametrize("T,d,d_out,bits_w,bits_a,gelu", [(300, 1024, 258, 4, 4, True),    # per-element stores
                                                          (520, 3072, 1024, 2, 4, False),  # row stores
                                                          (1024, 3072, 3072, 4, 8, True)])  # stream-K split
def test_gemm_bf16_output_is_rounded_fp32(T, d, d_out, bits_w, bits_a, gelu):
    from free_bit_quantization_amd import oq
    lin = synth.Linear(f"bf16out-{T}", T, d, d_out, 256, bits_w, bits_a, "student_t", "bf16", 10, 30.0, 0.5, 5,
                       10.0)
    x, Wm = synth.gen_linear(lin, 7, 0)
    x_idx, s, _ = P.check_activations(x, "bf16", lin.h, bits_a, rows=np.arange(4), want_x_rot=False)
    w_idx, w_norm, _ = P.check_weights(Wm, lin.h, bits_w)
    ca = P.library_codebook(d, bits_a)
    cw = P.library_codebook(d, bits_w)
    bias = torch.from_numpy(synth.gen_bias(d_out, 2)).cuda()
    epi = oq.OQ_EPI_GELU_ERF if gelu else oq.OQ_EPI_NONE
    split = T * d_out >= 1024 * 3072     # the third case takes the stream-K split
    y32 = P.run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bias, epilogue=epi, split=split)
    y16 = P.run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bias, epilogue=epi, split=split,
                     out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


# ---- full sizes, sampled outputs ------------------------------------------------


_sample_rows = P.sample_rows


# every token of every linear; the oracle works through the rows in chunks


def test_full_flux_qkv_w4a4():
    run_linear(W["flux_qkv_w4a4"].linears[0])


def test_full_flux_mlp_w2a4_chain():
    # the down projection takes the GPU's own GELU output; the whole chain
    # against the all-oracle chain (the oracle's indices everywhere) is reported
    up, down = W["flux_mlp_w2a4"].linears
    y_up = run_linear(up, index=0)
    x_down = y_up.cpu().numpy()
    _, W_down = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    y = run_linear(down, index=1, x=x_down, W_=W_down, x_dtype="f32")
    _chain_against_all_oracle(up, down, W_down, y)


def _chain_against_all_oracle(up, down, W_down, y, nrows=128):
    from oracle import quant
    rows = P.sample_rows(up.T, nrows)
    x, W_up = synth.gen_linear(up, 0, 0)
    pu, su, _, _ = P.rotation(up.d_in, up.h, 0)
    pdn, sdn, _, _ = P.rotation(down.d_in, down.h, 0)
    ca, cw = P.library_codebook(up.d_in, up.bits_a), P.library_codebook(up.d_in, up.bits_w)
    cda, cdw = P.library_codebook(down.d_in, down.bits_a), P.library_codebook(down.d_in, down.bits_w)
    ia, s_a, _, _ = quant.quantize_activations(x.astype(np.float64)[rows], pu, su, up.h, ca.th)
    iw, n_w, _, _ = quant.quantize_weights(W_up.astype(np.float64), pu, su, up.h, cw.th)
    h = quant.dequantized_product(ia, s_a, iw, n_w, ca.c, cw.c, gelu=True)
    ia2, s2, _, _ = quant.quantize_activations(h, pdn, sdn, down.h, cda.th)
    iw2, n2, _, _ = quant.quantize_weights(W_down.astype(np.float64), pdn, sdn, down.h, cdw.th)
    y_o = quant.dequantized_product(ia2, s2, iw2, n2, cda.c, cdw.c)
    err = P.rel_frob(y.float().cpu().numpy()[rows], y_o)
    P.log(f"[chain] GPU chain vs all-oracle chain: rel Frobenius {err:.3e} over {len(rows)} rows (information)")
    assert np.isfinite(err) and err <= 2e-2, err


def test_full_flux_mlp_w2a4_chain_bf16_hidden():
    up, down = W["flux_mlp_w2a4"].linears
    h16 = run_linear(up, index=0, out_dtype=torch.bfloat16)
    x_down = h16.float().cpu().numpy()
    _, W_down = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    run_linear(down, index=1, x=x_down, W_=W_down, x_dtype="bf16")


def test_full_wan_ffn_w4a4():
    run_linear(W["wan_ffn_w4a4"].linears[0])


@pytest.mark.parametrize("k", range(8))
def test_full_flux_block_w4a8(k):
    run_linear(W["flux_block_w4a8_b2"].linears[k], index=k)


def test_full_flux_qkv_split_every_tile():
    # the split entry point on the full FLUX QKV shape (its plan takes whole
    # tiles: a tail of 136 tiles of 24 stages), every output row checked
    run_linear(W["flux_qkv_w4a4"].linears[0], split=True)


# ---- the GELU epilogue against fp64 GELU of the GPU's own pre-activation -------


@pytest.mark.parametrize("T,d,n,bits_w,bits_a,split", [(300, 1024, 520, 2, 4, False), (4608, 3072, 1024, 2, 4, True),
                                                       (129, 3072, 517, 4, 8, False)])
def test_gelu_epilogue_matches_fp64_gelu_of_the_gpu_output(T, d, n, bits_w, bits_a, split):
    # the same inputs through the GEMM with and without the GELU epilogue:
    # GELU_fp64(y_none) must equal y_gelu to 1e-6 relative (absolute floor
    # 1e-6 * max|y| near zero, where GELU(y) ~ y / 2 carries y's rounding)
    from free_bit_quantization_amd import oq
    from oracle import quant
    lin = synth.Linear(f"gelu-{T}", T, d, n, 256, bits_w, bits_a, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0)
    x, Wm = synth.gen_linear(lin, 4, 0)
    x_idx, s, _ = P.check_activations(x, "bf16", 256, bits_a, rows=np.arange(4), want_x_rot=False)
    w_idx, w_norm, _ = P.check_weights(Wm, 256, bits_w)
    ca, cw = P.library_codebook(d, bits_a), P.library_codebook(d, bits_w)
    bias = torch.from_numpy(synth.gen_bias(n, 2)).cuda()
    y0 = P.run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bias, split=split,
                    workspace=oq.qlinear_workspace(T, n, d, bits_a, bits_w) if split else None)
    y1 = P.run_gemm(x_idx, s, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=bias, epilogue=oq.OQ_EPI_GELU_ERF,
                    split=split, workspace=oq.qlinear_workspace(T, n, d, bits_a, bits_w) if split else None)
    torch.cuda.synchronize()
    g = quant.gelu_erf(y0.cpu().numpy().astype(np.float64))
    got = y1.cpu().numpy().astype(np.float64)
    floor = 1e-6 * float(np.max(np.abs(g)))
    rel = np.abs(got - g) / np.maximum(np.abs(g), floor)
    P.log(f"[gelu] max relative difference {rel.max():.3e} over {got.size} outputs")
    assert rel.max() <= 1e-6
    # special and far values through the bias: +-inf, NaN, +-20, +-13.5, +-0
    special = np.array([np.inf, -np.inf, np.nan, 20.0, -20.0, 13.5, -13.5, 0.0, -0.0], dtype=np.float32)
    b2 = bias.clone()
    b2[:special.size] = torch.from_numpy(special).cuda()
    z0 = P.run_gemm(x_idx[:1], s[:1] * 1e-30, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=b2)
    z1 = P.run_gemm(x_idx[:1], s[:1] * 1e-30, w_idx, w_norm, d, bits_a, bits_w, ca.c, cw.c, bias=b2,
                    epilogue=oq.OQ_EPI_GELU_ERF)
    torch.cuda.synchronize()
    gz = quant.gelu_erf(z0.cpu().numpy().astype(np.float64))[0, :special.size]
    gotz = z1.cpu().numpy().astype(np.float64)[0, :special.size]
    with np.errstate(invalid="ignore"):
        ok = np.where(np.isfinite(gz), np.abs(gotz - gz) <= 1e-6 * np.maximum(np.abs(gz), 1e-30),
                      (gotz == gz) | (np.isnan(gotz) & np.isnan(gz)))
    P.log(f"[gelu] special values {special.tolist()} -> {gotz.tolist()} (fp64 {gz.tolist()})")
    assert ok.all()


# ---- launch geometry: the result does not depend on how the launch is cut --------


def test_rotate_quantize_launch_geometry_invariance():
    # 4096 tokens run with 12 wavefronts per workgroup, 2048 tokens with 8
    # (the plan switches at 3072): the rows they share are bit-identical, as
    # are 100 tokens (fewer tokens than workgroups)
    from free_bit_quantization_amd import oq
    lin = W["flux_qkv_w4a4"].linears[0]
    x, _ = synth.gen_linear(lin, 2, 0, T=4096)
    perm, sign, pd, sd = P.rotation(3072, 256, 0)
    for bits in (4, 8):
        th = P.library_codebook(3072, bits).th
        xd = P.to_device(x, "bf16")
        outs = [oq.oq_rotate_quantize_act(xd[:n].contiguous(), 256, pd, sd, th, bits, want_x_rot=True)
                for n in (4096, 2048, 100)]
        torch.cuda.synchronize()
        for (xi, s_, xr), n in zip(outs[1:], (2048, 100)):
            assert torch.equal(xi, outs[0][0][:n]) and torch.equal(s_, outs[0][1][:n])
            assert torch.equal(xr, outs[0][2][:n])


def test_gemm_launch_geometry_invariance():
    # the same rows in a launch of 18 x 36 tiles and of 2 x 36 tiles (other
    # grid, other tile-to-workgroup map): bit-identical whole-tile outputs
    lin = W["flux_qkv_w4a4"].linears[0]
    x, Wm = synth.gen_linear(lin, 6, 0)
    x_idx, s, _ = P.check_activations(x, "bf16", 256, 4, rows=np.arange(4), want_x_rot=False)
    w_idx, w_norm, _ = P.check_weights(Wm, 256, 4)
    cb = P.library_codebook(3072, 4)
    y_all = P.run_gemm(x_idx, s, w_idx, w_norm, 3072, 4, 4, cb.c, cb.c)
    y_few = P.run_gemm(x_idx[:512].contiguous(), s[:512].contiguous(), w_idx, w_norm, 3072, 4, 4, cb.c, cb.c)
    torch.cuda.synchronize()
    assert torch.equal(y_all[:512], y_few)


# ---- the workgroup kernel's binary search (no search grid fits) ------------------


@pytest.mark.parametrize("d,h,dtype", [(1024, 256, "bf16"), (12288, 256, "f32"), (256, 16, "f32")])
def test_rotate_quantize_binary_search_without_grid(d, h, dtype):
    # thresholds with two of them closer than the guard band allows for a
    # grid cell: the host builds no grid, and the workgroup kernel searches
    # the thresholds by bisection (the path with G = 0), still certified
    from free_bit_quantization_amd import oq
    from oracle import quant
    rng = np.random.default_rng(d + 1)
    th = P.library_codebook(d, 4).th.copy()
    th[9] = th[8] * (1.0 + 3e-6)          # a gap of 3e-6 relative: below 2.2 guard radii
    assert np.all(np.diff(th) > 0) and np.all(np.diff(th.astype(np.float32)) > 0)
    perm, sign, pd, sd = P.rotation(d, h, 0)
    x = rng.standard_t(3, size=(70, d)).astype(np.float32)
    # a quarter of the coordinates near the close pair, in the rotated basis
    from oracle import rpbh
    z = rpbh.rotate(x.astype(np.float64), perm, sign, h)
    nrm = np.linalg.norm(z, axis=1, keepdims=True)
    mask = rng.random(z.shape) < 0.1
    zm = th[8] * nrm * (1.0 + rng.choice([-1e-6, 1e-6, 2e-6, 4e-6], z.shape))
    # rescale the other coordinates so the row keeps its norm: the placed
    # coordinates then sit at u = th[8] (1 + e) up to the input's rounding
    rest2 = np.sum(np.where(mask, 0.0, z) ** 2, axis=1, keepdims=True)
    alpha = np.sqrt((nrm ** 2 - np.sum(np.where(mask, zm, 0.0) ** 2, axis=1, keepdims=True)) / rest2)
    z = np.where(mask, zm, alpha * z)
    xb = rpbh.rotate(z, np.arange(d), np.ones(d, dtype=np.int8), h)
    x2 = np.empty_like(xb)
    x2[:, perm] = sign[None, :] * xb
    x2 = x2.astype(np.float32)
    if dtype == "bf16":
        x2 = synth.bf16_round(x2)
    xd = P.to_device(x2, dtype)
    xi, s_, _ = oq.oq_rotate_quantize_act(xd, h, pd, sd, th, 4)
    torch.cuda.synchronize()
    ia, s_o, _, u_o = quant.quantize_activations(xd.float().cpu().numpy().astype(np.float64), perm, sign, h, th)
    gi = quant.unpack(xi.cpu().numpy(), 4, d)
    n, nin, nout = P.index_mismatches(gi, ia, u_o, th)
    near = np.min(np.abs(u_o[:, :, None] - th[None, None, 8:10]), axis=2) < (1e-4 if dtype == "f32" else 3e-2) * th[8]
    P.log(f"[bisect] d={d} {dtype}: mismatches {n} in band {nin} out of band {nout}; {int(near.sum())} near the pair")
    assert nout == 0 and near.sum() > 0
    assert np.max(np.abs(s_.cpu().numpy() - s_o) / s_o) <= P.REL_S


# ---- the certified guard under pressure: coordinates placed at the thresholds ----


@pytest.mark.parametrize("d,h,bits", [(1024, 256, 4), (3072, 256, 4), (2048, 64, 2), (3072, 256, 8)])
def test_guard_with_coordinates_at_thresholds(d, h, bits):
    # Rows built in the rotated basis: a quarter of the normalised coordinates
    # sit within +-3e-8 (relative) of a threshold, the rest are N(0, 1/d)
    # rescaled so each row has unit norm; x = R^T x_rot in fp64, rounded to fp32.
    # Many coordinates then fall inside the guard band (several per Hadamard
    # block), so the fp64 recheck decides them; the oracle judges every index.
    from oracle import rpbh
    rng = np.random.default_rng(d + h + bits)
    T = 64
    perm, sign, _, _ = P.rotation(d, h, 0, "rpbh")
    th = P.library_codebook(d, bits).th
    u = rng.standard_normal((T, d)) / np.sqrt(d)
    mask = rng.random((T, d)) < 0.25
    k = rng.integers(0, len(th), (T, d))
    delta = rng.choice(np.array([-3e-8, -1e-8, -1e-9, 1e-9, 1e-8, 3e-8]), (T, d))
    u = np.where(mask, th[k] * (1.0 + delta), u)
    placed = (u * mask) ** 2
    free = (u * ~mask) ** 2
    scale = np.sqrt((1.0 - placed.sum(axis=1)) / free.sum(axis=1))
    u = np.where(mask, u, u * scale[:, None])
    x_rot = 3.0 * u
    # inverse rotation: R = B D P with B symmetric, so x[perm] = sign * (B x_rot)
    z = rpbh.rotate(x_rot, np.arange(d), np.ones(d, dtype=np.int8), h)   # B x_rot
    x = np.empty_like(z)
    x[:, perm] = sign[None, :] * z
    x = x.astype(np.float32)
    _, _, rep = P.check_activations(x, "f32", h, bits, want_x_rot=False, name=f"guard-{d}-{h}-{bits}")
    _assert_act(rep)
    # the case has to reach the guard: count coordinates of the oracle's exact
    # rotation that lie within 1e-6 of a threshold
    xo = rpbh.rotate(x.astype(np.float64), perm, sign, h)
    uo = xo / np.linalg.norm(xo, axis=1, keepdims=True)
    near = np.min(np.abs(uo[:, :, None] - th[None, None, :]), axis=2) < 1e-6
    assert near.sum() > T * d // 20, near.sum()
