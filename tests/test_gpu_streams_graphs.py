"""The hot path under HIP graph capture and on concurrent streams.

The library allocates nothing, issues no memset and never synchronises on the
launch path, so rotate-quantize + GEMM can be captured into a graph (launch
overhead gone for serving loops) and run on several streams at once.  Every
replay is compared bit for bit with the eager result, with other eager work
between replays."""

import numpy as np
import pytest

from free_bit_quantization_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _setup(T=520, d=1024, n=777, h=256, seed=0):
    from free_bit_quantization_amd import oq
    lin = synth.Linear("g", T, d, n, h, 4, 4, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0)
    x, W = synth.gen_linear(lin, seed, 0)
    perm, sign = oq.oq_build_rpbh(d, h, 0)
    c, th, _ = oq.oq_lloyd_max(d, 4)
    pd, sd = torch.from_numpy(perm).cuda(), torch.from_numpy(sign).cuda()
    w_idx, w_norm = oq.oq_quantize_weights(torch.from_numpy(W).cuda(), h, pd, sd, th, 4)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    return oq, lin, xt, pd, sd, c, th, w_idx, w_norm


def test_graph_capture_replays_match_eager():
    oq, lin, xt, pd, sd, c, th, w_idx, w_norm = _setup()
    T, d, n = lin.T, lin.d_in, lin.d_out
    x_idx = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty(T, device="cuda")
    y = torch.empty((T, n), device="cuda")
    bias = torch.from_numpy(synth.gen_bias(n, 1)).cuda()

    def step(stream):
        oq.oq_rotate_quantize_act(xt, lin.h, pd, sd, th, 4, x_idx=x_idx, s=s, stream=stream)
        oq.oq_qlinear(x_idx, s, w_idx, w_norm, d, c, 4, c, 4, bias=bias, epilogue=oq.OQ_EPI_GELU_ERF, y=y,
                      stream=stream)

    step(None)
    torch.cuda.synchronize()
    y_ref, i_ref, s_ref = y.clone(), x_idx.clone(), s.clone()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step(cap)              # warm the capture stream outside the graph
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        x_idx.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x_idx, i_ref), f"replay {rep}: indices differ"
        assert torch.equal(s, s_ref), f"replay {rep}: norms differ"
        assert torch.equal(y, y_ref), f"replay {rep}: outputs differ"
        # eager work between replays
        step(None)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)


def test_concurrent_streams_match_sequential():
    oq, lin, xt, pd, sd, c, th, w_idx, w_norm = _setup(T=700, d=3072, n=1030, seed=3)
    T, d, n = lin.T, lin.d_in, lin.d_out
    xt2 = torch.flip(xt, dims=[0]).contiguous()
    outs = []
    for x_in in (xt, xt2):
        xi, s, _ = oq.oq_rotate_quantize_act(x_in, lin.h, pd, sd, th, 4)
        outs.append(oq.oq_qlinear(xi, s, w_idx, w_norm, d, c, 4, c, 4))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    res = [None, None]
    for rep in range(3):
        for k, (st, x_in) in enumerate(zip(streams, (xt, xt2))):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                xi = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
                s = torch.empty(T, device="cuda")
                yy = torch.empty((T, n), device="cuda")
                oq.oq_rotate_quantize_act(x_in, lin.h, pd, sd, th, 4, x_idx=xi, s=s, stream=st)
                oq.oq_qlinear(xi, s, w_idx, w_norm, d, c, 4, c, 4, y=yy, stream=st)
                res[k] = yy
        torch.cuda.synchronize()
        for k in range(2):
            assert torch.equal(res[k], outs[k]), f"stream {k} rep {rep} differs"
