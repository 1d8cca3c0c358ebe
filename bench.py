#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 hot path on one MI355X.

Main line (the JSON `value`): the MXFP4 W4A4 layer M=4096 N=8192 K=8192.
One step = quantize the fp32 activations X [4096, 8192] to MXFP4 + quantize
the fp32 weights W [8192, 8192] to MXFP4 + the W4A4 GEMM (bf16 out).
value = 2*M*N*K / step time, in TFLOPS.  Inputs are resident in HBM before
timing; two input sets (804 MB) alternate so that the 256 MB last-level cache
cannot hold a step's inputs.  Per-kernel durations come from HIP events
recorded on the stream the kernels run on.

Secondary measurements (same JSON line, `secondary`): the W4A16 GEMV
N=K=8192 at M = 1, 8, 16 (GB/s, weights rotated over 16 copies), the NVFP4
quantize + GEMM 2048x28672x8192 and the fused dynamic-quantize grouped GEMM
(8 experts, N=4096, K=14336, 8192 tokens).

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
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
GEMM_KERNEL = "k_gemm_mx"
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


class EvTimer:
    """Accumulates durations of regions bracketed by HIP events on a stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, {}

    def region(self, name):
        torch = self.torch
        tm = self

        class _R:
            def __enter__(self_):
                self_.s = torch.cuda.Event(enable_timing=True)
                self_.e = torch.cuda.Event(enable_timing=True)
                self_.s.record(tm.stream)

            def __exit__(self_, *a):
                self_.e.record(tm.stream)
                tm.pairs.setdefault(name, []).append((self_.s, self_.e))
        return _R()

    def mean_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(s.elapsed_time(e) for s, e in p) / max(len(p), 1)


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
    stream = torch.cuda.current_stream(dev)

    def step(i, tm=None):
        x, wt, aq, bq = sets[i % 2]
        if tm is None:
            mx.mx_quantize(x, out=aq)
            mx.mx_quantize(wt, out=bq)
            mx.mx_gemm(aq, bq, out=c)
            return
        with tm.region("quant_x"):
            mx.mx_quantize(x, out=aq)
        with tm.region("quant_w"):
            mx.mx_quantize(wt, out=bq)
        with tm.region("gemm"):
            mx.mx_gemm(aq, bq, out=c)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    tm = EvTimer(torch, stream)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    g_ms = tm.mean_ms("gemm")
    qx_ms, qw_ms = tm.mean_ms("quant_x"), tm.mean_ms("quant_w")
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
                     "kernel": GEMM_KERNEL, "flops_per_launch": flops, "avg_launch_ms": g_ms},
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
    reps = 16   # 16 weight copies x 35.7 MB rotate past the last-level cache
    ws = [mx.mx_quantize(wt) for _ in range(reps)]
    del wt
    out = {}
    stream = torch.cuda.current_stream(dev)
    for M in W.GEMV_M:
        x = torch.from_numpy(d["x"][:M]).to(torch.bfloat16).to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        for i in range(2 * reps):
            mx.mx_gemv(x, ws[i % reps], out=y)
        torch.cuda.synchronize()
        n = max(args.gemv_iters, reps)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for i in range(n):
            mx.mx_gemv(x, ws[i % reps], out=y)
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / n
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
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    tm = EvTimer(torch, stream)
    for it in range(1 + args.side_iters):
        t = tm if it else None
        for name, fn in (("quant_x", lambda: mx.mx_quantize(x, "nvfp4", out=aq, workspace=ws)),
                         ("quant_w", lambda: mx.mx_quantize(wt, "nvfp4", out=bq, workspace=ws)),
                         ("gemm", lambda: mx.mx_gemm(aq, bq, out=c))):
            if t is None:
                fn()
            else:
                with t.region(name):
                    fn()
    torch.cuda.synchronize()
    g = tm.mean_ms("gemm")
    flops = 2.0 * M * N * K
    qw = tm.mean_ms("quant_w")
    qw_bytes = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4   # amax pass + quantize pass
    return {"gemm_avg_ms": g, "gemm_TFLOPS": flops / (g * 1e-3) / 1e12,
            "gemm_frac_fp16_mfma_peak": flops / (g * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
            "gemm_frac_fp4_peak": flops / (g * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "quant_x_avg_ms": tm.mean_ms("quant_x"), "quant_w_avg_ms": qw,
            "quant_w_GB/s_two_reads": qw_bytes / (qw * 1e-3) / 1e9}


def bench_grouped(args, torch, mx, W):
    w = W.C5
    G, N, K, T = w.experts, w.N, w.K, w.M
    dev = torch.device("cuda:0")
    d = W.make(w)
    wq = mx.mx_quantize(torch.from_numpy(d["w"].reshape(G * N, K)).to(dev))
    x = torch.from_numpy(d["x"]).to(torch.bfloat16).to(dev)
    offs = torch.from_numpy(d["offsets"]).to(dev)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    wsz = T * K // 2 + T * K // 32 + 4096
    wsp = torch.empty(wsz, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    tm = EvTimer(torch, stream)
    for it in range(1 + args.side_iters):
        if it == 0:
            mx.mx_gemm(x, wq, N=N, out=y, groups=G, offsets=offs, workspace=wsp)
        else:
            with tm.region("fused"):
                mx.mx_gemm(x, wq, N=N, out=y, groups=G, offsets=offs, workspace=wsp)
    torch.cuda.synchronize()
    ms = tm.mean_ms("fused")
    flops = 2.0 * T * N * K
    return {"avg_ms": ms, "TFLOPS": flops / (ms * 1e-3) / 1e12, "frac_fp4_peak": flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "note": "one mx_gemm call: MXFP4 quantization of the bf16 tokens + grouped W4A4 GEMM"}


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only-main", action="store_true", help="skip secondary measurements and the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--gemv-iters", type=int, default=200)
    ap.add_argument("--side-iters", type=int, default=10)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); --gpus {args.gpus} is not "
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
        torch.cuda.empty_cache()
        log("secondary: NVFP4 quantize + GEMM")
        sec["nvfp4_2048x28672x8192"] = bench_nvfp4(args, torch, mx, W)
        torch.cuda.empty_cache()
        log("secondary: fused dynamic-quantize grouped GEMM")
        sec["grouped_8x4096x14336_T8192"] = bench_grouped(args, torch, mx, W)
        torch.cuda.empty_cache()
        out["secondary"] = sec
        if not args.no_cpu:
            log("cpu baseline (oracle)")
            out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
