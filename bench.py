#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 hot path on one MI355X.

Main line (the JSON `value`): the MXFP4 W4A4 layer M=4096 N=8192 K=8192.
One step = quantize the fp32 activations X [4096, 8192] to MXFP4 + quantize
the fp32 weights W [8192, 8192] to MXFP4 + the W4A4 GEMM (bf16 out).
value = 2*M*N*K / step time, in TFLOPS.  Inputs are resident in HBM before
timing; two input sets (804 MB) alternate so that the 256 MB last-level cache
cannot hold a step's inputs.  The timed steps replay HIP graphs (two steps,
one per input set, per graph launch; checked to reproduce the eager result).
The default 200 warmup steps (about 45 ms) let the clock settle under load;
after only 5 (1 ms) the timed steps run about 8 % slower.  Per-kernel
durations come from HIP events around graphs of back-to-back launches of
that kernel, on the stream they run on.

Secondary measurements (same JSON line, `secondary`): the W4A16 GEMV
N=K=8192 at M = 1, 8, 16 (GB/s, weights rotated over 16 copies), the NVFP4
quantize + GEMM 2048x28672x8192, the fused dynamic-quantize grouped GEMM
(8 experts, N=4096, K=14336, 8192 tokens), the routed expert layer
around it (4096 tokens, top-2: route, gathered quantize, grouped GEMM,
combine), the fused RMSNorm + quantize, and MXFP8 / MXFP6 products on the
4096x8192x8192 shape (FP8 x FP4, FP8 x FP8, FP6 x FP6), and the
quantization variants (16-element E8M0 blocks, the OCP floor rule, naive
per-tensor FP4, ...) with the reconstruction SNR of each.

cpu_baseline: the CPU oracle (numpy, fp64) on a bounded sub-problem of the
same step, timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 W4A4 GEMM TFLOPS + W4A16 GEMV GB/s on 1 MI355X, % of roofline"
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
GEMM_KERNEL = "k_gemm_mx_k256"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "microscaling_fp4_quantization_mx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, kernel_files):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(kernel_files):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def capture(torch, fn, reps=1):
    """A HIP graph of `reps` calls of fn (all launches on the capture stream).
    The step is launch-bound from Python (a few tens of microseconds of host
    work per call), so timed work replays graphs instead of calling eagerly."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                  # eager warm-up call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps_in_graph, replays=5):
    """Average duration of one captured call: HIP events around `replays`
    replays on the stream the graph runs on."""
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(replays):
        g.replay()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (replays * reps_in_graph)


def bench_main(args, torch, mx, W):
    w = W.C3
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    log(f"generating inputs for {w.name}")
    d = W.make(w)
    sets = []
    for i in range(2):   # two resident input sets alternate between steps
        x = torch.from_numpy(d["x"]).to(dev)
        wt = torch.from_numpy(d["w"]).to(dev)
        sets.append((x, wt, mx.empty_quantized(M, K, "mxfp4", dev), mx.empty_quantized(N, K, "mxfp4", dev)))
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def step(i):
        x, wt, aq, bq = sets[i % 2]
        mx.mx_quantize(x, out=aq)
        mx.mx_quantize(wt, out=bq)
        mx.mx_gemm(aq, bq, out=c)

    # Graphs: one per input set (single steps) and one holding two consecutive
    # steps (set 0 then set 1), which halves the per-launch gap between steps;
    # every step still quantizes both inputs and runs the GEMM.  A replay must
    # reproduce the eager result exactly.
    step(0)
    torch.cuda.synchronize()
    c_eager = c.clone()
    graphs = [capture(torch, lambda i=i: step(i)) for i in range(2)]
    pair = capture(torch, lambda: (step(0), step(1)))
    for g in (graphs[1], graphs[0], pair, graphs[0]):
        c.zero_()
        g.replay()
        torch.cuda.synchronize()
        if g is pair:
            ok_pair = torch.equal(c, c_eager)   # step(1) on set 1 equals step(0) on set 0 (same data)
    if not torch.equal(c, c_eager) or not ok_pair:
        raise RuntimeError("graph replay of the step differs from the eager step")

    def run(n):   # n consecutive steps, alternating input sets
        for _ in range(n // 2):
            pair.replay()
        if n % 2:
            graphs[0].replay()

    run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    del graphs, pair

    # per-kernel durations: events around graphs of back-to-back launches that
    # alternate between the two input sets (each set's fp32 inputs alone fill
    # about half of the last-level cache)
    R = 5

    def alt(fn):
        return lambda: [fn(*sets[i]) for i in (0, 1)]
    qx_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_quantize(x, out=aq)), R), 2 * R, replays=20)
    qw_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_quantize(wt, out=bq)), R), 2 * R, replays=20)
    g_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_gemm(aq, bq, out=c)), R), 2 * R, replays=20)
    flops = 2.0 * M * N * K
    qx_bytes = M * K * 4 + M * K // 2 + M * K // 32
    qw_bytes = N * K * 4 + N * K // 2 + N * K // 32
    gemm_bytes = (M + N) * (K // 2 + K // 32) + M * N * 2
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    traffic = load_traffic("mxfp4_gemm_4096x8192x8192_counters.txt", ["gemm_mxfp4.hip", "mx_device.h"])
    res = {
        "value": flops / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step,
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / PEAK_FP4_TFLOPS, "traffic": traffic,
                     "kernel": GEMM_KERNEL, "flops_per_launch": flops, "algorithmic_bytes_per_launch": gemm_bytes,
                     "avg_launch_ms": g_ms},
        "kernels": {
            "quantize_x": {"avg_ms": qx_ms, "GB/s": qx_bytes / (qx_ms * 1e-3) / 1e9, "bytes": qx_bytes,
                           "frac_hbm": qx_bytes / (qx_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "quantize_w": {"avg_ms": qw_ms, "GB/s": qw_bytes / (qw_ms * 1e-3) / 1e9, "bytes": qw_bytes,
                           "frac_hbm": qw_bytes / (qw_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "gemm": {"avg_ms": g_ms, "TFLOPS": gemm_tflops, "bytes": gemm_bytes},
        },
    }
    del sets
    torch.cuda.empty_cache()
    return res, d


def bench_gemv(args, torch, mx, W):
    w = W.C2
    N, K = w.N, w.K
    dev = torch.device("cuda:0")
    d = W.make(w)
    wt = torch.from_numpy(d["w"]).to(dev)
    reps = 16   # 16 weight copies x 35.7 MB rotate past the 256 MB last-level cache
    ws = [mx.mx_quantize(wt) for _ in range(reps)]
    del wt
    out = {}
    for M in W.GEMV_M:
        x = torch.from_numpy(d["x"][:M]).to(torch.bfloat16).to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

        def batch():
            for i in range(reps):
                mx.mx_gemv(x, ws[i], out=y)
        g = capture(torch, batch, max(1, args.gemv_iters // reps))
        ms = time_graph(torch, g, reps * max(1, args.gemv_iters // reps))
        byt = N * K // 2 + N * K // 32 + 2 * M * K + 2 * M * N
        gbs = byt / (ms * 1e-3) / 1e9
        out[f"M={M}"] = {"avg_ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "bytes": byt,
                         "TFLOPS": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
    return out


def bench_nvfp4(args, torch, mx, W):
    w = W.C4
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    d = W.make(w)
    x = torch.from_numpy(d["x"]).to(dev)
    wt = torch.from_numpy(d["w"]).to(dev)
    aq = mx.empty_quantized(M, K, "nvfp4", dev)
    bq = mx.empty_quantized(N, K, "nvfp4", dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    R = max(1, args.side_iters)
    qx = time_graph(torch, capture(torch, lambda: mx.mx_quantize(x, "nvfp4", out=aq, workspace=wsp), R), R)
    qw = time_graph(torch, capture(torch, lambda: mx.mx_quantize(wt, "nvfp4", out=bq, workspace=wsp), R), R)
    g = time_graph(torch, capture(torch, lambda: mx.mx_gemm(aq, bq, out=c), R), R, replays=2)
    flops = 2.0 * M * N * K
    qw_bytes = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4   # amax pass + quantize pass
    return {"gemm_avg_ms": g, "gemm_TFLOPS": flops / (g * 1e-3) / 1e12,
            "gemm_frac_fp16_mfma_peak": flops / (g * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
            "gemm_frac_fp4_peak": flops / (g * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "quant_x_avg_ms": qx, "quant_w_avg_ms": qw,
            "quant_w_GB/s_two_reads": qw_bytes / (qw * 1e-3) / 1e9}


def bench_wide(args, torch, mx, W):
    """MXFP8 / MXFP6 pairs on the 4096 x 8192 x 8192 product: quantize the bf16
    activations and fp32 weights to the pair's formats, then the GEMM."""
    w = W.WIDE
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    d = W.make(w)
    x = torch.from_numpy(d["x"]).to(torch.bfloat16).to(dev)
    wt = torch.from_numpy(d["w"]).to(dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    R = max(1, args.side_iters)
    res = {}
    for fa, fb in W.WIDE_PAIRS:
        aq = mx.empty_quantized(M, K, fa, dev)
        bq = mx.empty_quantized(N, K, fb, dev)
        qx = time_graph(torch, capture(torch, lambda: mx.mx_quantize(x, fa, out=aq), R), R)
        mx.mx_quantize(wt, fb, out=bq)
        g = time_graph(torch, capture(torch, lambda: mx.mx_gemm(aq, bq, out=c), R), R, replays=2)
        flops = 2.0 * M * N * K
        tf = flops / (g * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if "mxfp8" in (fa + fb) else PEAK_FP4_TFLOPS
        qbytes = M * K * 2 + M * K * mx.element_bits(fa) // 8 + M * K // 32
        res[f"{fa}_x_{fb}"] = {"gemm_avg_ms": g, "gemm_TFLOPS": tf, "gemm_peak_TFLOPS": peak, "gemm_frac": tf / peak,
                               "quant_x_bf16_avg_ms": qx, "quant_x_GB/s": qbytes / (qx * 1e-3) / 1e9}
        del aq, bq
    return res


def bench_variants(args, torch, mx, W):
    """The emulation variants on the 4096 x 8192 fp32 activations (outlier
    columns): quantize time and rate of each scheme, and the reconstruction
    SNR (dB) of its GPU dequantized output against the input (the accuracy
    measure of the pages' emulation demo; the error sums are measurement only)."""
    w = W.C3
    dev = torch.device("cuda:0")
    d = W.make(w)
    x = torch.from_numpy(d["x"]).to(dev)
    M, K = x.shape
    R = max(1, args.side_iters)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    x64 = x.double()
    sig = float((x64 * x64).sum())
    res = {}
    schemes = [("mxfp4_k32_ceil", "mxfp4", {}), ("mxfp4_k32_floor_ocp", "mxfp4", {"rule": "floor"}),
               ("mxfp4_k16_e8m0", "mxfp4_k16", {}), ("mxfp4_k16_e8m0_tensor_scale", "mxfp4_k16", {"static_global": 0.75}),
               ("nvfp4_k16_e4m3", "nvfp4", {}), ("fp4_per_tensor_naive", "fp4_tensor", {}),
               ("mxfp8_e4m3", "mxfp8_e4m3", {}), ("mxfp6_e2m3", "mxfp6_e2m3", {})]
    for name, fmt, kw in schemes:
        q = mx.empty_quantized(M, K, fmt, dev)
        t = time_graph(torch, capture(torch, lambda: mx.mx_quantize(x, fmt, out=q, workspace=ws, **kw), R), R)
        y = mx.mx_dequantize(q)
        err = float(((x64 - y.double()) ** 2).sum())
        bits = mx.element_bits(fmt)
        qbytes = M * K * 4 + M * K * bits // 8 + (0 if q.scales is None else q.scales.numel())
        res[name] = {"quant_avg_ms": t, "quant_GB/s": qbytes / (t * 1e-3) / 1e9,
                     "snr_db": 10.0 * __import__("math").log10(sig / err) if err > 0 else None}
        del q, y
    return res


def bench_grouped(args, torch, mx, W):
    w = W.C5
    G, N, K, T = w.experts, w.N, w.K, w.M
    dev = torch.device("cuda:0")
    d = W.make(w)
    wq = mx.mx_quantize(torch.from_numpy(d["w"].reshape(G * N, K)).to(dev))
    x = torch.from_numpy(d["x"]).to(torch.bfloat16).to(dev)
    offs = torch.from_numpy(d["offsets"]).to(dev)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    wsz = T * K // 2 + T * K // 32 + 4096   # >= mx_workspace_bytes for the dynamic A operand
    wsp = torch.empty(wsz, dtype=torch.uint8, device=dev)
    R = max(1, args.side_iters)
    ms = time_graph(torch, capture(torch, lambda: mx.mx_gemm(x, wq, N=N, out=y, groups=G, offsets=offs,
                                                             workspace=wsp), R), R, replays=3)
    flops = 2.0 * T * N * K
    return {"avg_ms": ms, "TFLOPS": flops / (ms * 1e-3) / 1e12, "frac_fp4_peak": flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "note": "one mx_gemm call: MXFP4 quantization of the bf16 tokens + grouped W4A4 GEMM"}


def bench_moe(args, torch, mx, W):
    """Routed expert layer: route (top-2 of 8) + gathered MXFP4 quantize of the
    bf16 tokens + grouped W4A4 GEMM (bf16 y) + weighted combine, one graph."""
    w = W.MOE
    T, G, N, K, k = w.M, w.experts, w.N, w.K, W.MOE_TOPK
    dev = torch.device("cuda:0")
    d = W.make(w)
    ids, tw = W.topk_routing(T, G, k)
    wq = mx.mx_quantize(torch.from_numpy(d["w"].reshape(G * N, K)).to(dev))
    x = torch.from_numpy(d["x"]).to(torch.bfloat16).to(dev)
    idt, twt = torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev)
    P = T * k
    bufs = {"offsets": torch.empty(G + 1, dtype=torch.int32, device=dev),
            "dest_row": torch.empty(P, dtype=torch.int32, device=dev),
            "src_token": torch.empty(P, dtype=torch.int32, device=dev),
            "route_ws": torch.empty(4096, dtype=torch.uint8, device=dev),
            "aq": mx.empty_quantized(P, K, "mxfp4", dev),
            "y": torch.empty(P, N, dtype=torch.bfloat16, device=dev),
            "out": torch.empty(T, N, dtype=torch.bfloat16, device=dev)}
    R = max(1, args.side_iters)
    ms = time_graph(torch, capture(torch, lambda: mx.moe_forward(x, idt, twt, wq, G, N, bufs=bufs), R), R, replays=3)
    flops = 2.0 * P * N * K
    return {"avg_ms": ms, "TFLOPS": flops / (ms * 1e-3) / 1e12, "frac_fp4_peak": flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "note": f"{T} tokens, top-{k} of {G} experts, N={N}, K={K}: route + gathered quantize + grouped GEMM + combine"}


def bench_rmsnorm(args, torch, mx, W):
    """RMSNorm fused with MXFP4 (and static-scale NVFP4) quantization of bf16
    tokens [8192, 14336] (the grouped workload's activations); two inputs
    alternate so the last-level cache cannot hold them."""
    w = W.C5
    T, K = w.M, w.K
    dev = torch.device("cuda:0")
    d = W.make(w)
    xs = [torch.from_numpy(d["x"]).to(torch.bfloat16).to(dev) for _ in range(2)]
    gamma = torch.ones(K, dtype=torch.float32, device=dev)
    res = {}
    for fmt, k, sg in (("mxfp4", 32, None), ("nvfp4", 16, 0.01)):
        outs = [mx.empty_quantized(T, K, fmt, dev) for _ in range(2)]
        R = max(1, args.side_iters)
        ms = time_graph(torch, capture(torch, lambda: [mx.mx_rmsnorm_quantize(xs[i], gamma, 1e-6, fmt, outs[i], sg)
                                                       for i in (0, 1)], R), 2 * R)
        byt = T * K * 2 + K * 4 + T * K // 2 + T * K // k
        res[fmt] = {"avg_ms": ms, "GB/s": byt / (ms * 1e-3) / 1e9, "frac_hbm": byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                    "bytes": byt}
    return res


def cpu_baseline(d):
    """The oracle, as it stands, on a bounded sub-problem of the same step:
    X rows 0..1023 and W rows 0..4095 (both quantized) and their GEMM."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    mr, nr, K = 1024, 4096, d["x"].shape[1]
    x, w = d["x"][:mr], d["w"][:nr]
    t0 = time.perf_counter()
    ca, sa = O.mxfp4_quantize(x)
    cb, sb = O.mxfp4_quantize(w)
    y = O.gemm(O.dequantize("mxfp4", ca, sa), O.dequantize("mxfp4", cb, sb), out="bf16")
    dt = time.perf_counter() - t0
    assert y.shape == (mr, nr)
    return {"value": 2.0 * mr * nr * K / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"sub-problem {mr}x{nr}x{K} of the step (quantize X rows, quantize W rows, fp64 GEMM); "
                      f"{dt:.1f} s; quantization single-threaded numpy, GEMM via BLAS with {threads} threads",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the clock needs tens of milliseconds of load to settle")
    ap.add_argument("--only-main", action="store_true", help="skip secondary measurements and the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--gemv-iters", type=int, default=200)
    ap.add_argument("--side-iters", type=int, default=10)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import microscaling_fp4_quantization_mx_amd as mx
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mx.lib()
    if args.calib_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("calibration copy: 512 MiB read + 512 MiB written by one elementwise kernel")
        del src, dst
    res, d = bench_main(args, torch, mx, W)
    log(f"main: {res['value']:.1f} TFLOPS per step, GEMM {res['roofline']['achieved']:.1f} TFLOPS")
    out = {"metric": METRIC, "value": res["value"], "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
           "config": {"workload": W.C3.name, "M": W.C3.M, "N": W.C3.N, "K": W.C3.K,
                      "step": "quantize X fp32->MXFP4 + quantize W fp32->MXFP4 + W4A4 GEMM (fp32 accumulate, bf16 out)",
                      "parallelism": "single GPU"},
           "roofline": res["roofline"], "kernels": res["kernels"]}
    if not args.only_main:
        sec = {}
        log("secondary: W4A16 GEMV")
        sec["w4a16_gemv_8192x8192"] = bench_gemv(args, torch, mx, W)
        g1 = sec["w4a16_gemv_8192x8192"]["M=1"]
        sec["w4a16_gemv_8192x8192"]["roofline_M1"] = {"bound": "hbm", "achieved": g1["GB/s"], "peak": PEAK_HBM_GBS,
                                                       "unit": "GB/s", "frac": g1["frac_hbm"],
                                                       "traffic": load_traffic("gemv_m1_8192x8192_counters.txt",
                                                                               ["gemv.hip", "mx_device.h"])}
        g16 = sec["w4a16_gemv_8192x8192"]["M=16"]
        sec["w4a16_gemv_8192x8192"]["roofline_M16"] = {"bound": "hbm", "achieved": g16["GB/s"], "peak": PEAK_HBM_GBS,
                                                        "unit": "GB/s", "frac": g16["frac_hbm"],
                                                        "traffic": load_traffic("gemv_m16_8192x8192_counters.txt",
                                                                                ["gemv.hip", "mx_device.h"])}
        torch.cuda.empty_cache()
        log("secondary: NVFP4 quantize + GEMM")
        sec["nvfp4_2048x28672x8192"] = bench_nvfp4(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: MXFP8 / MXFP6 GEMM pairs")
        sec["mx_wide_gemm_4096x8192x8192"] = bench_wide(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: quantization variants and reconstruction SNR")
        sec["variants_4096x8192_fp32"] = bench_variants(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: fused dynamic-quantize grouped GEMM")
        sec["grouped_8x4096x14336_T8192"] = bench_grouped(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: fused RMSNorm + FP4 quantize")
        sec["rmsnorm_quantize_8192x14336_bf16"] = bench_rmsnorm(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: routed expert layer (top-2)")
        sec["moe_top2_8x4096x14336_T4096"] = bench_moe(args, torch, mx, W)
        torch.cuda.empty_cache()
        out["secondary"] = sec
        if not args.no_cpu:
            log("cpu baseline (oracle)")
            out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
