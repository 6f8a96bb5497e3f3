"""The hot path under HIP graph capture and on concurrent streams.

No entry point allocates, issues a memset or synchronises on the launch path,
so rotate-quantize + GEMM can be captured into a graph (launch overhead gone
for serving loops) and run on several streams at once.  The split GEMM
(oq_qlinear_splitk) exchanges partial tiles through a caller-owned workspace:
a graph records its workspace, and launches that run at the same time use
different workspaces.  Every replay is compared bit for bit with the eager
result, with other eager work (split launches on another stream and
workspace, and on the capture stream's own workspace) between replays."""

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


def _setup(T=520, d=3072, n=777, h=256, seed=0):
    from free_bit_quantization_amd import oq
    lin = synth.Linear("g", T, d, n, h, 4, 4, "student_t", "bf16", 10, 30.0, 0.5, 5, 10.0)
    x, W = synth.gen_linear(lin, seed, 0)
    perm, sign = oq.oq_build_rpbh(d, h, 0)
    c, th, _ = oq.oq_lloyd_max(d, 4)
    pd, sd = torch.from_numpy(perm).cuda(), torch.from_numpy(sign).cuda()
    w_idx, w_norm = oq.oq_quantize_weights(torch.from_numpy(W).cuda(), h, pd, sd, th, 4)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    return oq, lin, xt, pd, sd, c, th, w_idx, w_norm


@pytest.mark.parametrize("split", [False, True])
def test_graph_capture_replays_match_eager(split):
    oq, lin, xt, pd, sd, c, th, w_idx, w_norm = _setup()
    T, d, n = lin.T, lin.d_in, lin.d_out
    x_idx = torch.empty((T, d // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty(T, device="cuda")
    y = torch.empty((T, n), device="cuda")
    bias = torch.from_numpy(synth.gen_bias(n, 1)).cuda()
    ws_graph = oq.qlinear_workspace(T, n, d, 4, 4) if split else None
    ws_other = oq.qlinear_workspace(T, n, d, 4, 4) if split else None
    if split:
        assert ws_graph is not None   # 12 tiles of 24 K stages: the split is taken

    def step(stream, xi, ss, yy, ws):
        oq.oq_rotate_quantize_act(xt, lin.h, pd, sd, th, 4, x_idx=xi, s=ss, stream=stream)
        if split:
            oq.oq_qlinear_splitk(xi, ss, w_idx, w_norm, d, c, 4, c, 4, ws, bias=bias, epilogue=oq.OQ_EPI_GELU_ERF,
                                 y=yy, stream=stream)
        else:
            oq.oq_qlinear(xi, ss, w_idx, w_norm, d, c, 4, c, 4, bias=bias, epilogue=oq.OQ_EPI_GELU_ERF, y=yy,
                          stream=stream)

    step(None, x_idx, s, y, ws_graph)
    torch.cuda.synchronize()
    y_ref, i_ref, s_ref = y.clone(), x_idx.clone(), s.clone()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step(cap, x_idx, s, y, ws_graph)     # warm the capture stream outside the graph
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step(cap, x_idx, s, y, ws_graph)
    torch.cuda.synchronize()
    other = torch.cuda.Stream()
    xi2 = torch.empty_like(x_idx)
    s2 = torch.empty_like(s)
    y2 = torch.empty_like(y)
    for rep in range(3):
        y.fill_(float("nan"))
        x_idx.zero_()
        s.zero_()
        y2.fill_(float("nan"))
        torch.cuda.synchronize()
        # the replay and an eager launch on another stream and workspace, at once
        g.replay()
        with torch.cuda.stream(other):
            step(other, xi2, s2, y2, ws_other)
        torch.cuda.synchronize()
        assert torch.equal(x_idx, i_ref), f"replay {rep}: indices differ"
        assert torch.equal(s, s_ref), f"replay {rep}: norms differ"
        assert torch.equal(y, y_ref), f"replay {rep}: outputs differ"
        assert torch.equal(y2, y_ref), f"replay {rep}: the concurrent eager launch differs"
        # eager work on the graph's own workspace between replays (ordered)
        step(None, x_idx, s, y, ws_graph)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)


@pytest.mark.parametrize("split", [False, True])
def test_concurrent_streams_match_sequential(split):
    oq, lin, xt, pd, sd, c, th, w_idx, w_norm = _setup(T=700, d=3072, n=1030, seed=3)
    T, d, n = lin.T, lin.d_in, lin.d_out
    xt2 = torch.flip(xt, dims=[0]).contiguous()
    wss = [oq.qlinear_workspace(T, n, d, 4, 4) if split else None for _ in range(2)]
    if split:
        assert wss[0] is not None

    def gemm(xi, s, yy=None, stream=None, ws=None):
        if split:
            return oq.oq_qlinear_splitk(xi, s, w_idx, w_norm, d, c, 4, c, 4, ws, y=yy, stream=stream)
        return oq.oq_qlinear(xi, s, w_idx, w_norm, d, c, 4, c, 4, y=yy, stream=stream)

    outs = []
    for x_in in (xt, xt2):
        xi, s, _ = oq.oq_rotate_quantize_act(x_in, lin.h, pd, sd, th, 4)
        outs.append(gemm(xi, s, ws=wss[0]))
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
                gemm(xi, s, yy=yy, stream=st, ws=wss[k])
                res[k] = yy
        torch.cuda.synchronize()
        for k in range(2):
            assert torch.equal(res[k], outs[k]), f"stream {k} rep {rep} differs"
