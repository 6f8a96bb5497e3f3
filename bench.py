#!/usr/bin/env python
"""Benchmark of the OrbitQuant quantized linear on one MI355X.

One step = the whole hot path on one batch: rotate-and-quantize of the
token activations (oq_rotate_quantize_act) followed by the codebook GEMM
(oq_qlinear_splitk with a workspace allocated before timing; --whole-tiles:
oq_qlinear), on the FLUX.1-like double-stream QKV linear (4608 tokens,
3072 -> 9216, W4A4, h = 256).  Weights are quantized once, offline,
before timing.  Inputs are resident in HBM when the timed region starts;
the activation batches rotate through a ring of buffers larger than the
256 MB Infinity Cache so the rotate-quantize kernel reads from HBM.

Prints one JSON line.  Per-kernel durations come from HIP events recorded
on the launch stream around every kernel of the timed steps.  With --sweep it
prints one line per linear of every workload instead (throughput and roofline
fractions only); with --modulation one line per AdaLN modulation projection
(the INT4 round-to-nearest W4A16 kernel, HBM roofline); with --mlp the
chained MLP pair, once with an fp32 and once with a bf16 hidden state.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this
# bench (FETCH_SIZE x 2, WRITE_SIZE x 1: the copy-kernel calibration), valid only
# for the kernel source they were taken on (sha256 prefix); otherwise null.
MEASURED_TRAFFIC = {
    "free_bit_quantization_amd/csrc/qlinear.hip": ("79ccc4d384d96871", 113.53e6, 169.91e6),
    "free_bit_quantization_amd/csrc/rotate_quantize.hip": ("9dfb6acdbef78b69", 28.68e6, 7.23e6),
}


TRAFFIC_SOURCE = ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of this bench, profiles/flux_qkv_w4a4_kernels.md "
                  "(null when the kernel source changed since)")


def traffic_of(src: str):
    import hashlib
    entry = MEASURED_TRAFFIC.get(src)
    if entry is None:
        return None
    digest = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
    if digest != entry[0]:
        return None
    return entry[1] + entry[2]


def cpu_baseline(lin, x, Wm, perm, sign, c_a, th_a, c_w, th_w, target_s: float = 12.0):
    """The fp64 oracle on the host cores, on a bounded sample of tokens of the
    same workload, in the same unit as the GPU value (TFLOP/s of the layer)."""
    import numpy as np
    from oracle import quant
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    # offline weight step (not timed, as on the GPU)
    iw, n_w, _, _ = quant.quantize_weights(Wm.astype(np.float64), perm, sign, lin.h, th_w)

    def run(n):
        xs = x[:n].astype(np.float64)
        t0 = time.perf_counter()
        ia, s, _, _ = quant.quantize_activations(xs, perm, sign, lin.h, th_a)
        quant.dequantized_product(ia, s, iw, n_w, c_a, c_w)
        return time.perf_counter() - t0

    t_probe = run(32)
    n = int(min(lin.T, max(32, 32 * target_s / max(t_probe, 1e-3))))
    # repeat the sample until about target_s of CPU time has been measured
    t, reps = 0.0, 0
    while reps == 0 or (t < target_s and reps < 64):
        t += run(n)
        reps += 1
    flops = 2.0 * n * reps * lin.d_in * lin.d_out
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {lin.T} tokens x {reps} passes (rotate-quantize + fp64 dequantized product), {t:.1f} s",
            "tokens_per_s": n * reps / t}


def measure_linear(lin, index, steps, warmup, ring_mb, dev, split=True):
    """Time rotate-quantize + codebook GEMM of one linear (inputs resident in HBM).
    split: the GEMM through oq_qlinear_splitk with a workspace allocated before
    timing (stream-K tail where the shape takes it), else oq_qlinear."""
    import torch
    from free_bit_quantization_amd import oq, synth

    T, K, N, h = lin.T, lin.d_in, lin.d_out, lin.h
    x, Wm = synth.gen_linear(lin, 0, index)
    perm, sign = oq.oq_build_rpbh(K, h, 0)
    c_a, th_a, _ = oq.oq_lloyd_max(K, lin.bits_a)
    c_w, th_w, _ = oq.oq_lloyd_max(K, lin.bits_w)
    pd = torch.from_numpy(perm).to(dev)
    sd = torch.from_numpy(sign).to(dev)
    xt = torch.from_numpy(x).to(dev)
    if lin.act_dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    Wd = torch.from_numpy(Wm).to(dev)
    w_idx, w_norm = oq.oq_quantize_weights(Wd, h, pd, sd, th_w, lin.bits_w)
    del Wd

    # ring of activation batches (distinct buffers) larger than the Infinity Cache
    nring = max(1, math.ceil(ring_mb * 1e6 / (xt.numel() * xt.element_size())))
    ring = [xt] + [torch.roll(xt, shifts=i * 7, dims=0).contiguous() for i in range(1, nring)]
    x_idx = torch.empty((T, K * lin.bits_a // 8), dtype=torch.uint8, device=dev)
    s = torch.empty(T, dtype=torch.float32, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    epi = oq.OQ_EPI_GELU_ERF if lin.epilogue == "gelu" else oq.OQ_EPI_NONE
    ws = oq.qlinear_workspace(T, N, K, lin.bits_a, lin.bits_w) if split else None

    def gemm():
        if split:
            oq.oq_qlinear_splitk(x_idx, s, w_idx, w_norm, K, c_a, lin.bits_a, c_w, lin.bits_w, ws, epilogue=epi, y=y,
                                 stream=stream)
        else:
            oq.oq_qlinear(x_idx, s, w_idx, w_norm, K, c_a, lin.bits_a, c_w, lin.bits_w, epilogue=epi, y=y,
                          stream=stream)

    def step(i):
        oq.oq_rotate_quantize_act(ring[i % nring], h, pd, sd, th_a, lin.bits_a, x_idx=x_idx, s=s, stream=stream)
        gemm()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        oq.oq_rotate_quantize_act(ring[i % nring], h, pd, sd, th_a, lin.bits_a, x_idx=x_idx, s=s, stream=stream)
        e[1].record(stream)
        gemm()
        e[2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    total_ms = start.elapsed_time(end)
    ms_step = total_ms / steps
    t_rq = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t_ql = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    # medians of the per-step intervals (the model card reports warm medians)
    med = lambda v: sorted(v)[len(v) // 2]
    medians = {"step": med([e[0].elapsed_time(e[2]) for e in ev]),
               "rotate_quant": med([e[0].elapsed_time(e[1]) for e in ev]),
               "qlinear": med([e[1].elapsed_time(e[2]) for e in ev])}
    es = xt.element_size()
    rq_bytes = T * K * es + T * K * lin.bits_a // 8 + 4 * T       # read x, write indices and s
    flops = 2.0 * T * K * N
    r = dict(T=T, K=K, N=N, h=h, es=es, nring=nring, ms_step=ms_step, t_rq=t_rq, t_ql=t_ql, t_wall=t_wall,
             rq_bytes=rq_bytes, flops=flops, rq_gbs=rq_bytes / (t_rq * 1e-3) / 1e9,
             ql_tflops=flops / (t_ql * 1e-3) / 1e12, value=flops / (ms_step * 1e-3) / 1e12,
             entry="oq_qlinear_splitk" if ws is not None else "oq_qlinear", ws_bytes=0 if ws is None else ws.numel(),
             medians=medians,
             inputs=(x, Wm, perm, sign, c_a, th_a, c_w, th_w))
    return r


def measure_mlp(up, down, hidden, steps, warmup, ring_mb, dev, folded=False):
    """Time the chained MLP pair: rotate-quantize x, up GEMM with the GELU
    epilogue into the hidden state h, rotate-quantize h, down GEMM.  h is
    fp32 or bf16 (the up GEMM rounds its output to nearest even).  folded:
    the down rotation's permutation folded into the up projection's rows
    (oq_fold_permutation, offline), so the down rotate-quantize gathers with
    the identity permutation."""
    import torch
    from free_bit_quantization_amd import oq, synth

    T, K, H, N, hb = up.T, up.d_in, up.d_out, down.d_out, up.h
    assert down.d_in == H and down.T == T
    x, W_up = synth.gen_linear(up, 0, 0)
    _, W_dn = synth.gen_linear(down, 0, 1, T=1, need_act=False)
    rot = {}
    for d in (K, H):
        pm, sg = oq.oq_build_rpbh(d, hb, 0)
        rot[d] = (torch.from_numpy(pm).to(dev), torch.from_numpy(sg).to(dev))
    cb = {(d, b): oq.oq_lloyd_max(d, b) for d in (K, H) for b in {up.bits_a, up.bits_w, down.bits_a, down.bits_w}}
    wq = []
    for lin, Wm in ((up, W_up), (down, W_dn)):
        Wd = torch.from_numpy(Wm).to(dev)
        wq.append(oq.oq_quantize_weights(Wd, hb, *rot[lin.d_in], cb[(lin.d_in, lin.bits_w)][1], lin.bits_w))
        del Wd
    bias_up = torch.from_numpy(synth.gen_bias(H, 3)).to(dev)
    rq_down_tables = rot[H]
    if folded:
        wi, wn, bias_up = oq.oq_fold_permutation(wq[0][0], wq[0][1], rot[H][0], K, up.bits_w, bias=bias_up)
        wq[0] = (wi, wn)
        rq_down_tables = (torch.arange(H, dtype=torch.int32, device=dev), rot[H][1])
    xt = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    nring = max(1, math.ceil(ring_mb * 1e6 / (xt.numel() * xt.element_size())))
    ring = [xt] + [torch.roll(xt, shifts=i * 7, dims=0).contiguous() for i in range(1, nring)]
    hd = torch.bfloat16 if hidden == "bf16" else torch.float32
    xi_u = torch.empty((T, K * up.bits_a // 8), dtype=torch.uint8, device=dev)
    s_u = torch.empty(T, dtype=torch.float32, device=dev)
    hbuf = torch.empty((T, H), dtype=hd, device=dev)
    xi_d = torch.empty((T, H * down.bits_a // 8), dtype=torch.uint8, device=dev)
    s_d = torch.empty(T, dtype=torch.float32, device=dev)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def kernels(i):
        yield lambda: oq.oq_rotate_quantize_act(ring[i % nring], hb, *rot[K], cb[(K, up.bits_a)][1], up.bits_a,
                                                x_idx=xi_u, s=s_u, stream=stream)
        yield lambda: oq.oq_qlinear(xi_u, s_u, wq[0][0], wq[0][1], K, cb[(K, up.bits_a)][0], up.bits_a,
                                    cb[(K, up.bits_w)][0], up.bits_w, bias=bias_up, epilogue=oq.OQ_EPI_GELU_ERF,
                                    y=hbuf, stream=stream)
        yield lambda: oq.oq_rotate_quantize_act(hbuf, hb, *rq_down_tables, cb[(H, down.bits_a)][1], down.bits_a,
                                                x_idx=xi_d, s=s_d, stream=stream)
        yield lambda: oq.oq_qlinear(xi_d, s_d, wq[1][0], wq[1][1], H, cb[(H, down.bits_a)][0], down.bits_a,
                                    cb[(H, down.bits_w)][0], down.bits_w, y=y, stream=stream)

    for i in range(warmup):
        for k in kernels(i):
            k()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        for j, k in enumerate(kernels(i)):
            k()
            ev[i][j + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    per = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j in range(4)]
    flops = 2.0 * T * K * H + 2.0 * T * H * N
    rq_down_bytes = T * H * hbuf.element_size() + T * H * down.bits_a // 8 + 4 * T
    return {"workload": "flux_mlp_chain", "hidden": hidden, "folded_permutation": folded,
            "tokens": T, "d_in": K, "d_hidden": H, "d_out": N,
            "bits_w": up.bits_w, "bits_a": up.bits_a, "h": hb, "hidden_bytes": T * H * hbuf.element_size(),
            "ms_per_step": round(ms_step, 5), "tokens_per_s": round(T / (ms_step * 1e-3), 1),
            "TFLOPs": round(flops / (ms_step * 1e-3) / 1e12, 2),
            "rq_up_ms": round(per[0], 5), "gemm_up_ms": round(per[1], 5), "rq_down_ms": round(per[2], 5),
            "gemm_down_ms": round(per[3], 5), "rq_down_GBps": round(rq_down_bytes / (per[2] * 1e-3) / 1e9, 1),
            "rq_down_frac_hbm": round(rq_down_bytes / (per[2] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "activation_ring_buffers": nring}


def measure_modulation(lin, steps, warmup, ring_mb, dev):
    """Time the W4A16 modulation projection (INT4 RTN weights streamed from HBM).

    The packed weights rotate through a ring of copies larger than the
    Infinity Cache.  The kernel is a few microseconds long, shorter than a
    host launch, so the stream is held by a spin kernel while every timed
    launch is enqueued; one pair of HIP events then brackets the launches
    running back to back on the GPU (per-launch events would add their own
    overhead to a kernel this short)."""
    import torch
    from free_bit_quantization_amd import oq, synth

    T, K, N, g = lin.T, lin.d_in, lin.d_out, lin.group
    x, Wm = synth.gen_modulation(lin, seed=0)
    xt = torch.from_numpy(x).to(dev)
    xt = xt.to(torch.bfloat16) if lin.act_dtype == "bf16" else xt.to(torch.float16)
    Wd = torch.from_numpy(Wm).to(dev)
    q, sc = oq.oq_quantize_weights_int4(Wd, g)
    del Wd
    wbytes = q.numel() + sc.numel() * 4
    nring = max(1, math.ceil(ring_mb * 1e6 / wbytes))
    ring = [(q, sc)] + [(q.clone(), sc.clone()) for _ in range(1, nring)]
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        oq.oq_linear_w4a16(xt, ring[i % nring][0], ring[i % nring][1], g, y=y, stream=stream)
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(1.0e7 + 2.0e5 * steps))   # >= 5 ms + 100 us per launch
        e0.record(stream)
        for i in range(steps):
            oq.oq_linear_w4a16(xt, ring[i % nring][0], ring[i % nring][1], g, y=y, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) / steps)
    reps.sort()
    t_avg = reps[1]   # median of three back-to-back runs
    alg = N * K // 2 + N * (K // g) * 4 + T * K * xt.element_size() + T * N * 4
    return dict(T=T, K=K, N=N, group=g, nring=nring, t_ms=t_avg, t_runs=reps,
                bytes=alg, gbs=alg / (t_avg * 1e-3) / 1e9)


def modulation_line(name, lin, r):
    return {"workload": name, "linear": lin.name, "kernel": "oq_linear_w4a16 (w4a_kernel)",
            "tokens": r["T"], "d_in": r["K"], "d_out": r["N"], "group": r["group"], "act_dtype": lin.act_dtype,
            "ms": round(r["t_ms"], 5), "ms_runs": [round(t, 5) for t in r["t_runs"]],
            "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                         "algorithmic": f"N*K/2 + N*(K/group)*4 + T*K*2 + T*N*4 = {r['bytes']} B"},
            "weight_ring_buffers": r["nring"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: the GPU clock ramps over the first ~60 ms of work")
    ap.add_argument("--workload", default="flux_qkv_w4a4")
    ap.add_argument("--ring-mb", type=float, default=640.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="one line per linear of every workload (tokens/s, GB/s, TFLOP/s, roofline fractions)")
    ap.add_argument("--modulation", action="store_true",
                    help="one line per AdaLN modulation projection (INT4 RTN W4A16 kernel)")
    ap.add_argument("--mlp", action="store_true",
                    help="the chained FLUX-like MLP pair (rq, up GEMM + GELU, rq, down GEMM), one line with an "
                         "fp32 and one with a bf16 hidden state")
    ap.add_argument("--sweep-workloads", default="",
                    help="comma-separated workload names for --sweep (default: all)")
    ap.add_argument("--whole-tiles", action="store_true",
                    help="time the GEMM through oq_qlinear (whole tiles, no workspace) instead of oq_qlinear_splitk")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the layer is "
              "token-parallel; see the sharding design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from free_bit_quantization_amd import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.modulation:
        for name, lins in synth.modulation_workloads().items():
            for lin in lins:
                r = measure_modulation(lin, max(args.steps, 50), args.warmup, args.ring_mb, dev)
                print(json.dumps(modulation_line(name, lin, r)), flush=True)
        return

    if args.mlp:
        up, down = synth.workloads()["flux_mlp_w2a4"].linears
        for hidden in ("f32", "bf16"):
            for folded in (False, True):
                print(json.dumps(measure_mlp(up, down, hidden, args.steps, args.warmup, args.ring_mb, dev, folded)),
                      flush=True)
                torch.cuda.empty_cache()
        return

    if args.sweep:
        names = [n for n in args.sweep_workloads.split(",") if n] or synth.WORKLOAD_ORDER
        for name in names:
            for k, lin in enumerate(synth.workloads()[name].linears):
                r = measure_linear(lin, k, args.steps, args.warmup, args.ring_mb, dev, split=not args.whole_tiles)
                print(json.dumps({
                    "workload": name, "linear": lin.name, "tokens": r["T"], "d_in": r["K"], "d_out": r["N"],
                    "h": r["h"], "bits_w": lin.bits_w, "bits_a": lin.bits_a, "act_dtype": lin.act_dtype,
                    "epilogue": lin.epilogue, "tokens_per_s": round(r["T"] / (r["ms_step"] * 1e-3), 1),
                    "ms_per_step": round(r["ms_step"], 5),
                    "qlinear_entry": r["entry"],
                    "qlinear_TFLOPs": round(r["ql_tflops"], 2), "qlinear_ms": round(r["t_ql"], 5),
                    "qlinear_frac_fp16_peak": round(r["ql_tflops"] / FP16_MFMA_PEAK_TFLOPS, 4),
                    "rotate_quant_GBps": round(r["rq_gbs"], 1), "rotate_quant_ms": round(r["t_rq"], 5),
                    "rotate_quant_frac_hbm": round(r["rq_gbs"] / HBM_PEAK_GBS, 4)}), flush=True)
                del r
                torch.cuda.empty_cache()
        return

    wl = synth.workloads()[args.workload]
    lin = wl.linears[0]
    r = measure_linear(lin, 0, args.steps, args.warmup, args.ring_mb, dev, split=not args.whole_tiles)
    T, K, N, h = r["T"], r["K"], r["N"], r["h"]
    es, rq_bytes, flops = r["es"], r["rq_bytes"], r["flops"]
    ms_step, t_rq, t_ql = r["ms_step"], r["t_rq"], r["t_ql"]
    rq_gbs, ql_tflops, value = r["rq_gbs"], r["ql_tflops"], r["value"]
    nring, t_wall = r["nring"], r["t_wall"]
    x, Wm, perm, sign, c_a, th_a, c_w, th_w = r["inputs"]

    line = {
        "metric": "qlinear TFLOP/s + rotate-quant GB/s (frac of roofline), FLUX 3072-wide W4A4",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc; fp32 rotate",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {T} tokens, {K}->{N}, W{lin.bits_w}A{lin.bits_a}, h={h}, "
                               f"{lin.act_dtype} activations", "tokens": T, "d_in": K, "d_out": N, "h": h,
                   "bits_w": lin.bits_w, "bits_a": lin.bits_a, "activation_ring_buffers": nring},
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "qlinear_TFLOPs": round(ql_tflops, 2),
        "qlinear_ms": round(t_ql, 5),
        "rotate_quant_GBps": round(rq_gbs, 1),
        "rotate_quant_ms": round(t_rq, 5),
        "median_ms": {k: round(v, 5) for k, v in r["medians"].items()},
        "roofline": {"bound": "mfma", "achieved": round(ql_tflops, 2), "peak": FP16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ql_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic_of("free_bit_quantization_amd/csrc/qlinear.hip"), "traffic_unit": "bytes",
                     "traffic_source": TRAFFIC_SOURCE,
                     "kernel": (f"{r['entry']} (ql_kernel<{lin.bits_a},{lin.bits_w},"
                                + ("true>: whole-tile rounds + stream-K last round)" if r["ws_bytes"] else
                                   "false>: whole tiles)")),
                     "workspace_bytes": r["ws_bytes"], "algorithmic": f"2*T*K*N = {flops:.4g} flop"},
        "roofline_rotate_quant": {"bound": "hbm", "achieved": round(rq_gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(rq_gbs / HBM_PEAK_GBS, 4),
                                  "traffic": traffic_of("free_bit_quantization_amd/csrc/rotate_quantize.hip"),
                                  "traffic_unit": "bytes", "traffic_source": TRAFFIC_SOURCE,
                                  "kernel": "oq_rotate_quantize_act (rq_wave_kernel<8,bf16,4,3,768>)",
                                  "algorithmic": f"T*(K*{es} + K*{lin.bits_a}/8 + 4) = {rq_bytes} B"},
        "wall_s_timed": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(lin, x, Wm, perm, sign, c_a, th_a, c_w, th_w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
