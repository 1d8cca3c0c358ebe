#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 hot path on one MI355X.

Main line (the JSON `value`): the MXFP4 W4A4 layer M=4096 N=8192 K=8192.
One step = quantize the fp32 activations X [4096, 8192] to MXFP4 + quantize
the fp32 weights W [8192, 8192] to MXFP4 + the W4A4 GEMM (bf16 out).
value = 2*M*N*K / step time, in TFLOPS.  Inputs are resident in HBM before
timing; two input sets (804 MB) alternate so that the 256 MB last-level cache
cannot hold a step's inputs.  The timed steps replay HIP graphs (two steps,
one per input set, per graph launch; checked to reproduce the eager result).
Per-kernel durations come from HIP events around graphs of back-to-back
launches of each kernel, on the stream they run on; they are measured first
(about 45 ms of full-load work), which also lets the clock settle before the
warmup and timed steps (without it, 5 warmup steps leave the timed steps
about 8 % slower than 200 do).

Secondary measurements (same JSON line, `secondary`): the W4A16 GEMV
N=K=8192 at M = 1, 8, 16 (GB/s, weights rotated over 16 copies), the NVFP4
quantize + GEMM 2048x28672x8192, the fused dynamic-quantize grouped GEMM
(8 experts, N=4096, K=14336, 8192 tokens), the routed expert layer
around it (4096 tokens, top-2: route, gathered quantize, grouped GEMM,
combine), the fused RMSNorm + quantize, and MXFP8 / MXFP6 products on the
4096x8192x8192 shape (FP8 x FP4, FP8 x FP8, FP6 x FP6), the
quantization variants (16-element E8M0 blocks, the OCP floor rule, naive
per-tensor FP4, ...) with the reconstruction SNR of each, and the vendor
library's MXFP4 GEMM (hipBLASLt) on the headline shape beside libmx's.

Ceilings (`secondary.ceilings`): a plain streaming read of the GEMV's bytes
and plain copies, the practical bounds beside the 8 TB/s peak.

cpu_baseline: the CPU oracle (numpy, fp64) on the whole step, timed on this
host's cores.
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


# counter summary of the quantize kernels (X and W of the main step share one
# grid size, so the figure is their mean over the dispatches of that grid)
QSUM = "quantize_counters.txt"
QFILES = ["quantize.hip", "nv_codes.h", "mx_device.h"]


def kernel_counter(name, kernel_files, kernel, grid, field):
    """A derived figure (field, e.g. "mfma_busy_frac") of one kernel and grid
    from a committed summary written by --summarize-pmc, if it was taken on
    the current kernel source; else None."""
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
    # kernel: a name ("k_gemm_mx_k256": any instantiation) or a name with the
    # start of its template arguments ("k_quant_mx<float")
    prefixes = (f"mxk::{kernel}",) if "<" in kernel else (f"mxk::{kernel}<", f"mxk::{kernel}@")
    for k, v in kv.items():
        if k.startswith(prefixes) and k.endswith(f"@{grid}.{field}"):
            return float(v)
    return None


def summarize_trace(dirs, out_path, title, command):
    """Per kernel and grid: dispatch count and duration statistics from
    rocprofv3 kernel-trace CSVs."""
    import collections
    import csv
    import glob
    import statistics
    d = collections.defaultdict(list)
    for dd in dirs:
        for f in glob.glob(os.path.join(dd, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                grid = r["Grid_Size"] if "Grid_Size" in r else r["Grid_Size_X"]
                k = (r["Kernel_Name"].split("(")[0].replace("void ", ""), grid)
                d[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = [f"# {title}", "# Command (repository root, TMPDIR=/tmp, one MI355X):"]
    lines += [f"#   {c}" for c in command]
    lines += ["# Durations are End - Start per dispatch in microseconds (warm-up and graph-capture calls included).",
              f"{'kernel':60s} {'grid':>9s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>9s}"]
    for (name, grid), v in sorted(d.items()):
        # libmx's kernels, and the vendor library's GEMM timed beside them
        if not (name.startswith("mxk::") or "GEMM" in name or "Cijk" in name):
            continue
        lines.append(f"{name:60s} {grid:>9s} {len(v):6d} {sum(v) / len(v):9.2f} {statistics.median(v):9.2f} "
                     f"{min(v):9.2f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


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

    # Per-kernel durations first: events around graphs of back-to-back
    # launches that alternate between the two input sets (each set's fp32
    # inputs alone fill about half of the last-level cache).  These ~45 ms of
    # full-load work also let the clock settle before the warmup steps.
    R = 5

    def alt(fn):
        return lambda: [fn(*sets[i]) for i in (0, 1)]
    qx_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_quantize(x, out=aq)), R), 2 * R, replays=20)
    qw_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_quantize(wt, out=bq)), R), 2 * R, replays=20)
    g_ms = time_graph(torch, capture(torch, alt(lambda x, wt, aq, bq: mx.mx_gemm(aq, bq, out=c)), R), 2 * R, replays=20)

    run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    del graphs, pair

    flops = 2.0 * M * N * K
    qx_bytes = M * K * 4 + M * K // 2 + M * K // 32
    qw_bytes = N * K * 4 + N * K // 2 + N * K // 32
    gemm_bytes = (M + N) * (K // 2 + K // 32) + M * N * 2
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    gfiles = ["gemm_mxfp4.hip", "gemm_mx_tile.h", "gemm_tiles.h", "gemm_split.h", "mx_device.h"]
    gsum = "mxfp4_gemm_4096x8192x8192_counters.txt"
    traffic = kernel_counter(gsum, gfiles, "k_gemm_mx_k256", 131072, "hbm_bytes")
    res = {
        "value": flops / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step,
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / PEAK_FP4_TFLOPS, "traffic": traffic,
                     "kernel": GEMM_KERNEL, "flops_per_launch": flops, "algorithmic_bytes_per_launch": gemm_bytes,
                     "avg_launch_ms": g_ms,
                     "mfma_busy_frac": kernel_counter(gsum, gfiles, "k_gemm_mx_k256", 131072, "mfma_busy_frac"),
                     "clock_ghz_under_profiler": kernel_counter(gsum, gfiles, "k_gemm_mx_k256", 131072, "clock_ghz"),
                     "counters": f"profiles/{gsum}"},
        "kernels": {
            "quantize_x": {"avg_ms": qx_ms, "GB/s": qx_bytes / (qx_ms * 1e-3) / 1e9, "bytes": qx_bytes,
                           "frac_hbm": qx_bytes / (qx_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "traffic_mean_x_and_w": kernel_counter(QSUM, QFILES, "k_quant_mx<float", 1048576, "hbm_bytes"),
                           "counters": f"profiles/{QSUM}"},
            "quantize_w": {"avg_ms": qw_ms, "GB/s": qw_bytes / (qw_ms * 1e-3) / 1e9, "bytes": qw_bytes,
                           "frac_hbm": qw_bytes / (qw_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           "counters": f"profiles/{QSUM}"},
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
    # The same product on the vector ALU only: at K = 8224 (not a multiple
    # of 256) mx_gemv runs its dot2 kernel for every M, so these lines show
    # what the MFMA-free path reaches at M = 8 and 16 (0.4 % more K).
    K2 = K + 32
    w2 = torch.from_numpy(W.weights(N, K2)).to(dev)
    ws2 = [mx.mx_quantize(w2) for _ in range(reps)]
    del w2
    for M in (8, 16):
        x = torch.from_numpy(W.activations(M, K2)).to(torch.bfloat16).to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

        def batch2():
            for i in range(reps):
                mx.mx_gemv(x, ws2[i], out=y)
        g = capture(torch, batch2, max(1, args.gemv_iters // reps))
        ms = time_graph(torch, g, reps * max(1, args.gemv_iters // reps))
        byt = N * K2 // 2 + N * K2 // 32 + 2 * M * K2 + 2 * M * N
        out[f"M={M}_vector_alu_K{K2}"] = {"avg_ms": ms, "GB/s": byt / (ms * 1e-3) / 1e9,
                                          "frac_hbm": byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                          "note": "dot2 kernel (no matrix cores)"}
    del ws2
    # W8A16 / W6A16: the same product with MXFP8 E4M3 / MXFP6 E2M3 weights
    # (the dot2 kernel for every M; 2x / 1.5x the weight bytes of MXFP4)
    wt = torch.from_numpy(d["w"]).to(dev)
    for fmt, bits in (("mxfp8_e4m3", 8), ("mxfp6_e2m3", 6)):
        wsf = [mx.mx_quantize(wt, fmt) for _ in range(reps)]
        for M in (1, 16):
            x = torch.from_numpy(d["x"][:M]).to(torch.bfloat16).to(dev)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

            def batch3():
                for i in range(reps):
                    mx.mx_gemv(x, wsf[i], out=y)
            g = capture(torch, batch3, max(1, args.gemv_iters // reps))
            ms = time_graph(torch, g, reps * max(1, args.gemv_iters // reps))
            byt = N * K * bits // 8 + N * K // 32 + 2 * M * K + 2 * M * N
            out[f"{fmt}_M={M}"] = {"avg_ms": ms, "GB/s": byt / (ms * 1e-3) / 1e9,
                                   "frac_hbm": byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": byt}
        del wsf
    del wt
    for M, kern in ((1, "k_gemv_sk"), (8, "k_gemv_mf"), (16, "k_gemv_mf")):
        g = out[f"M={M}"]
        out[f"roofline_M{M}"] = {"bound": "hbm", "achieved": g["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": g["frac_hbm"],
                                 "traffic": kernel_counter("gemv_8192x8192_counters.txt", ["gemv.hip", "mx_expand.h", "mx_device.h"],
                                                           f"{kern}<{M}" if kern == "k_gemv_mf" else kern,
                                                           131072, "hbm_bytes")}
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
    # X (64 MiB of fp32) rotates over 8 copies (2 x the 256 MB last-level
    # cache), so each quantize reads it from HBM like the 940 MB weights do
    xs = [x] + [x.clone() for _ in range(7)]

    def quant_x_all():
        for xi in xs:
            mx.mx_quantize(xi, "nvfp4", out=aq, workspace=wsp)
    qx = time_graph(torch, capture(torch, quant_x_all, max(1, R // 8)), len(xs) * max(1, R // 8))
    del xs
    qw = time_graph(torch, capture(torch, lambda: mx.mx_quantize(wt, "nvfp4", out=bq, workspace=wsp), R), R)
    g = time_graph(torch, capture(torch, lambda: mx.mx_gemm(aq, bq, out=c), R), R, replays=2)
    flops = 2.0 * M * N * K
    qw_bytes = 2 * N * K * 4 + N * K // 2 + N * K // 16 + 4   # amax pass + quantize pass
    qx_bytes = 2 * M * K * 4 + M * K // 2 + M * K // 16 + 4
    return {"gemm_avg_ms": g, "gemm_TFLOPS": flops / (g * 1e-3) / 1e12,
            "gemm_frac_fp16_mfma_peak": flops / (g * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
            "gemm_frac_fp4_peak": flops / (g * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "quant_x_avg_ms": qx, "quant_x_GB/s_two_reads": qx_bytes / (qx * 1e-3) / 1e9, "quant_w_avg_ms": qw,
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
        gf = time_graph(torch, capture(torch, lambda: mx.mx_gemm(aq, bq, out=c, f8f6f4_matrix_cores=True), R), R,
                        replays=2)
        flops = 2.0 * M * N * K
        tf, tff = flops / (g * 1e-3) / 1e12, flops / (gf * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if "mxfp8" in (fa + fb) else PEAK_FP4_TFLOPS
        qbytes = M * K * 2 + M * K * mx.element_bits(fa) // 8 + M * K // 32
        res[f"{fa}_x_{fb}"] = {"exact_gemm_avg_ms": g, "exact_gemm_TFLOPS": tf,
                               "exact_gemm_frac_bf16_peak": tf / PEAK_F16_TFLOPS,
                               "f8f6f4_gemm_avg_ms": gf, "f8f6f4_gemm_TFLOPS": tff, "f8f6f4_gemm_peak_TFLOPS": peak,
                               "f8f6f4_gemm_frac": tff / peak,
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
    R = max(1, args.side_iters)
    # the binding sizes the workspace (codes of the quantized tokens; with the
    # fused kernel also its counters and partial tiles) with mx_workspace_bytes;
    # the two forms alternate over three rounds, each keeping its best round
    g2 = capture(torch, lambda: mx.mx_gemm(x, wq, N=N, out=y, groups=G, offsets=offs), R)
    g1 = capture(torch, lambda: mx.mx_gemm(x, wq, N=N, out=y, groups=G, offsets=offs, fused_quantize=True), R)
    ms, ms_fused = 1e30, 1e30
    for _ in range(3):
        ms = min(ms, time_graph(torch, g2, R, replays=3))
        ms_fused = min(ms_fused, time_graph(torch, g1, R, replays=3))
    del g1, g2
    flops = 2.0 * T * N * K
    return {"avg_ms": ms, "TFLOPS": flops / (ms * 1e-3) / 1e12, "frac_fp4_peak": flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS,
            "note": "one mx_gemm call: MXFP4 quantization of the bf16 tokens (its own launch) + grouped W4A4 GEMM",
            "fused_avg_ms": ms_fused, "fused_TFLOPS": flops / (ms_fused * 1e-3) / 1e12,
            "fused_note": "the same call with MX_GEMM_FUSED_QUANTIZE: quantization and GEMM in one persistent kernel"}


def route_ws_bytes(mx, experts):
    import ctypes
    e = ctypes.c_int32(experts)
    return int(mx.lib().mx_workspace_bytes(mx.MX_OP_MOE_ROUTE, ctypes.cast(ctypes.pointer(e), ctypes.c_void_p), 0))


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
            "route_ws": torch.empty(route_ws_bytes(mx, G), dtype=torch.uint8, device=dev),
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
    """The oracle, as it stands, on the whole step: quantize all of X and W
    (row chunks on a thread pool with one worker per host core, at most 16;
    the oracle's numpy steps release the GIL) and the fp64 GEMM (numpy's
    BLAS, on its own threads)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    cores = min(16, os.cpu_count() or 1)
    x, w = d["x"], d["w"]
    M, K = x.shape
    N = w.shape[0]

    def quantize(t):
        parts = [t[r:r + 128] for r in range(0, t.shape[0], 128)]
        with ThreadPoolExecutor(cores) as ex:
            outs = list(ex.map(O.mxfp4_quantize, parts))
        return np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs])
    t0 = time.perf_counter()
    ca, sa = quantize(x)
    cb, sb = quantize(w)
    y = O.gemm(O.dequantize("mxfp4", ca, sa), O.dequantize("mxfp4", cb, sb), out="bf16")
    dt = time.perf_counter() - t0
    assert y.shape == (M, N)
    return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"the whole step {M}x{N}x{K} (quantize X, quantize W, fp64 GEMM), not extrapolated; "
                      f"{dt:.1f} s; quantization on {cores} threads, GEMM in numpy's BLAS",
            "seconds": dt}


def bench_ceilings(args, torch, mx, W):
    """Practical ceilings beside the 8 TB/s peak: a plain streaming read of
    the GEMV's weight bytes (35.7 MB, rotating over 16 buffers so every read
    comes from HBM) and plain copies of the quantize inputs' sizes, by the
    measurement-only kernels of libmx_ceiling.so (16-byte loads, four in
    flight per lane); the best of 2, 4 and 8 workgroups per CU.  Beside the
    10.1 PF FP4 peak: the FP4 matrix-core rate of a register-only loop, and
    the LDS rate of 16-byte fragment reads."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "microscaling_fp4_quantization_mx_amd", "libmx_ceiling.so"))
    L.mxc_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.mxc_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    sink = torch.empty(256 * 8, dtype=torch.int32, device=dev)
    out = {}
    gemv_bytes = W.C2.N * W.C2.K // 2 + W.C2.N * W.C2.K // 32 + 2 * W.C2.K + 2 * W.C2.N
    nb = (gemv_bytes + 255) // 256 * 256
    bufs = [torch.ones(nb // 4, dtype=torch.int32, device=dev) for _ in range(16)]
    best = None
    for per_cu in (2, 4, 8):
        def f():
            st = torch.cuda.current_stream().cuda_stream     # the capturing stream
            for b in bufs:
                assert L.mxc_read(b.data_ptr(), nb, sink.data_ptr(), per_cu, st) == 0
        ms = time_graph(torch, capture(torch, f, 8), 16 * 8)
        gbs = nb / (ms * 1e-3) / 1e9
        best = max(best or 0.0, gbs)
    out["read_35.7MB_GB/s"] = best
    del bufs
    for name, nbytes in (("copy_128MiB_GB/s", 128 << 20), ("copy_256MiB_GB/s", 256 << 20)):
        src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        dsts = [torch.empty_like(src) for _ in range(2)]
        best = None
        for per_cu in (2, 4, 8):
            def f():
                st = torch.cuda.current_stream().cuda_stream
                for dd in dsts:
                    assert L.mxc_copy(src.data_ptr(), dd.data_ptr(), nbytes, per_cu, st) == 0
            ms = time_graph(torch, capture(torch, f, 4), 2 * 4)
            best = max(best or 0.0, 2 * nbytes / (ms * 1e-3) / 1e9)   # read + write
        out[name] = best
        del src, dsts
    # on-chip rates of the GEMM's K loop: the FP4 matrix cores with operands in
    # registers (two waves per SIMD), and 16-byte LDS fragment reads
    L.mxc_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.mxc_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    grid, iters = 512, 2000
    sinkf = torch.empty(grid * 256, dtype=torch.float32, device=dev)

    def fm():
        assert L.mxc_mfma(sinkf.data_ptr(), grid, iters, torch.cuda.current_stream().cuda_stream) == 0
    ms = time_graph(torch, capture(torch, fm, 4), 4)
    out["mfma_fp4_32x32x64_register_loop_TFLOPS"] = grid * 4 * iters * 4 * 131072.0 / (ms * 1e-3) / 1e12
    grid, iters = 256, 2000
    sinku = torch.empty(grid * 256, dtype=torch.int32, device=dev)

    def fl():
        assert L.mxc_lds(sinku.data_ptr(), grid, iters, torch.cuda.current_stream().cuda_stream) == 0
    ms = time_graph(torch, capture(torch, fl, 4), 4)
    lds_bytes = grid * 4 * iters * 8 * 1024.0
    out["lds_read_b128_TB/s"] = lds_bytes / (ms * 1e-3) / 1e12
    out["lds_read_b128_B_per_clk_per_CU_at_2.4GHz"] = lds_bytes / (ms * 1e-3) / 256 / 2.4e9
    del sinkf, sinku
    return out


def bench_vendor(args, torch, mx, W):
    """The vendor library's MXFP4 GEMM on the headline shape, for context:
    torch._scaled_mm on float4_e2m1fn_x2 operands with E8M0 scale bytes,
    which ROCm's torch hands to hipBLASLt (its kernel name is in the kernel
    trace summary).  Both GEMMs run on the same seeded random codes, eagerly
    and back to back (no graph: the library call is not captured), libmx
    through its C entry point with prebuilt arguments; HIP events on the
    current stream; the two alternate in rounds after a warm-up and each
    reports its best round (the clock settles over the first tens of
    milliseconds of load).  Every scale byte is 127 (2^0): the result then
    does not depend on the library's scale layout, and every fp32 partial sum
    of E2M1 products is exact (multiples of 1/4 below 2^22), so libmx's fp32
    output is the exact product; the bf16 outputs are compared with its
    round-to-nearest-even and its truncation."""
    import ctypes
    w = W.C3
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)
    sets = []
    for _ in range(2):
        a = mx.empty_quantized(M, K, "mxfp4", dev)
        b = mx.empty_quantized(N, K, "mxfp4", dev)
        for t in (a, b):
            t.codes.copy_(torch.randint(0, 256, t.codes.shape, dtype=torch.uint8, device=dev, generator=gen))
            t.scales.fill_(127)
        sets.append((a, b))
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def vendor(a, b):
        return torch._scaled_mm(a.codes.view(torch.float4_e2m1fn_x2), b.codes.view(torch.float4_e2m1fn_x2).t(),
                                a.scales.view(torch.float8_e8m0fnu).flatten(),
                                b.scales.view(torch.float8_e8m0fnu).flatten(), out_dtype=torch.bfloat16)
    out = {"library": "hipBLASLt through torch._scaled_mm (float4_e2m1fn_x2, E8M0 scales)",
           "shape": [M, N, K]}
    try:
        y = vendor(*sets[0])
    except Exception as ex:   # torch or library without MXFP4 support
        out["error"] = f"{type(ex).__name__}: {str(ex)[:200]}"
        return out
    exact = mx.mx_gemm(*sets[0], out_dtype=torch.float32)
    mx.mx_gemm(*sets[0], out=c)
    torch.cuda.synchronize()
    rne = exact.to(torch.bfloat16)
    trunc = (exact.view(torch.int32) & ~0xFFFF).view(torch.float32).to(torch.bfloat16)
    out["libmx_bf16_equals_rne_of_exact"] = bool(torch.equal(c, rne))
    out["vendor_bf16_equals_rne_of_exact_frac"] = float((y == rne).float().mean())
    out["vendor_bf16_equals_truncation_of_exact_frac"] = float((y == trunc).float().mean())
    del y, exact, rne, trunc
    stream = torch.cuda.current_stream()
    flops = 2.0 * M * N * K
    L = mx.lib()
    descs, cargs = [], []
    for a, b in sets:
        ad, bd = a.desc(), b.desc()
        g = mx.CMxGemmArgs()
        g.M, g.N, g.K = M, N, K
        g.a, g.b = ctypes.pointer(ad), ctypes.pointer(bd)
        g.c, g.c_dtype, g.ldc = c.data_ptr(), mx.MX_DT_BF16, N
        descs += [ad, bd]
        cargs.append(g)
    sp = stream.cuda_stream

    def libmx(i):
        assert L.mx_gemm(ctypes.byref(cargs[i % 2]), sp) == 0

    def vend(i):
        vendor(*sets[i % 2])
    reps = max(20, args.side_iters * 5)
    for i in range(200):          # about 60 ms of load before the first timed round
        libmx(i)
        vend(i)
    torch.cuda.synchronize()
    best = {}
    for _ in range(3):
        for name, fn in (("libmx", libmx), ("vendor", vend)):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for i in range(reps):
                fn(i)
            e.record(stream)
            torch.cuda.synchronize()
            best[name] = min(best.get(name, 1e30), s.elapsed_time(e) / reps)
    for name, ms in best.items():
        out[f"{name}_avg_ms"] = ms
        out[f"{name}_TFLOPS"] = flops / (ms * 1e-3) / 1e12
        out[f"{name}_frac_fp4_peak"] = flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS
    out["libmx_speedup_over_vendor"] = best["vendor"] / best["libmx"]
    del sets
    return out


SECONDARY = {
    "ceilings": (bench_ceilings, "ceilings"),
    "gemv": (bench_gemv, "w4a16_gemv_8192x8192"),
    "nvfp4": (bench_nvfp4, "nvfp4_2048x28672x8192"),
    "wide": (bench_wide, "mx_wide_gemm_4096x8192x8192"),
    "variants": (bench_variants, "variants_4096x8192_fp32"),
    "grouped": (bench_grouped, "grouped_8x4096x14336_T8192"),
    "rmsnorm": (bench_rmsnorm, "rmsnorm_quantize_8192x14336_bf16"),
    "moe": (bench_moe, "moe_top2_8x4096x14336_T4096"),
    "vendor": (bench_vendor, "vendor_mxfp4_gemm_4096x8192x8192"),
}
SECONDARY_NAMES = tuple(SECONDARY)


def summarize_pmc(dirs, out_path, title, command, kernel_files, algorithmic=None):
    """Turn rocprofv3 counter-collection CSVs (one directory per pass) into a
    committed summary: per kernel and grid, the mean of every counter per
    dispatch, the kernel time from the dispatch timestamps, and derived
    figures.  Calibration of the HBM byte counters: FETCH_SIZE x 2,
    WRITE_SIZE x 1 (KiB), measured on a 512 MiB elementwise copy."""
    import collections
    import csv
    import glob
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = (r["Kernel_Name"].split("(")[0].replace("void ", ""), r["Grid_Size"])
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] in ("GRBM_GUI_ACTIVE", "FETCH_SIZE"):
                    dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = [f"# {title}", "# Commands (repository root, TMPDIR=/tmp, one MI355X), one counter pass each:"]
    lines += [f"#   {c}" for c in command]
    lines += ["# Units: counters are means per dispatch.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the",
              "# kernel's cycles are GRBM_GUI_ACTIVE / 8 and its clock that / the dispatch time.  MFMA busy",
              "# fraction = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU x 4 /",
              "# (cycles x 1024) (quad-cycles per wave summed per SIMD); LDS busy = SQ_LDS_IDX_ACTIVE / (cycles x 256).",
              "# HBM bytes: FETCH_SIZE x 2 KiB and WRITE_SIZE x 1 KiB (calibrated on a 512 MiB copy).",
              "# For dispatches of a few microseconds GRBM_GUI_ACTIVE includes a fixed window around the kernel, so",
              "# the GRBM-derived clock and busy fractions are too high / too low there; the VALU issue fraction uses",
              "# the dispatch time instead: SQ_INSTS_VALU / (dispatch time x 2.4 GHz x 1024 SIMDs / 4).",
              f"# source_hash = sha256 of {', '.join(kernel_files)} (first 16 hex digits) when the counters were taken;",
              "# bench.py reports these figures only while the kernel source still has this hash.",
              f"source_hash={source_hash(kernel_files)}"]
    for (name, grid), cs in sorted(agg.items()):
        if not (name.startswith("mxk::") or "AUnaryFunctor" in name):   # library kernels and the calibration copy
            continue
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        t_us = sum(dur[(name, grid)]) / max(1, len(dur[(name, grid)]))
        lines.append(f"# {name} grid {grid}: {len(next(iter(cs.values())))} dispatches per pass, {t_us:.2f} us "
                     "per dispatch under the profiler")
        for c in sorted(m):
            lines.append(f"#   {c:34s} {m[c]:18.1f}")
        if "GRBM_GUI_ACTIVE" in m:
            cyc = m["GRBM_GUI_ACTIVE"] / 8
            lines.append(f"#   kernel cycles {cyc:.0f}, clock {cyc / (t_us * 1e3):.3f} GHz")
        key = f"{name}@{grid}"
        if "GRBM_GUI_ACTIVE" in m:
            cyc = m["GRBM_GUI_ACTIVE"] / 8
            lines.append(f"{key}.clock_ghz={cyc / (t_us * 1e3):.4f}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                lines.append(f"{key}.mfma_busy_frac={m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.4f}")
            if "SQ_ACTIVE_INST_VALU" in m:
                lines.append(f"{key}.valu_busy_frac={m['SQ_ACTIVE_INST_VALU'] * 4 / (cyc * 1024):.4f}")
            if "SQ_LDS_IDX_ACTIVE" in m:
                lines.append(f"{key}.lds_busy_frac={m['SQ_LDS_IDX_ACTIVE'] / (cyc * 256):.4f}")
            if "SQ_LDS_BANK_CONFLICT" in m:
                lines.append(f"{key}.lds_bank_conflict_frac={m['SQ_LDS_BANK_CONFLICT'] / (cyc * 256):.4f}")
            if "TA_TA_BUSY_sum" in m:
                lines.append(f"{key}.ta_busy_frac={m['TA_TA_BUSY_sum'] / (cyc * 256):.4f}")
        if "SQ_INSTS_VALU" in m:
            # issue slots: one wave instruction per 4 clocks per SIMD, 1024 SIMDs, at the 2.4 GHz peak clock
            # (an upper bound on the slots, so the fraction is a lower bound)
            lines.append(f"{key}.valu_insts={m['SQ_INSTS_VALU']:.0f}")
            lines.append(f"{key}.valu_issue_frac_at_2400MHz={m['SQ_INSTS_VALU'] / (t_us * 2400 * 256):.4f}")
        if "FETCH_SIZE" in m:
            lines.append(f"{key}.fetch_bytes={m['FETCH_SIZE'] * 2 * 1024:.0f}")
        if "WRITE_SIZE" in m:
            lines.append(f"{key}.write_bytes={m['WRITE_SIZE'] * 1024:.0f}")
        if "FETCH_SIZE" in m and "WRITE_SIZE" in m:
            hbm = m["FETCH_SIZE"] * 2 * 1024 + m["WRITE_SIZE"] * 1024
            lines.append(f"{key}.hbm_bytes={hbm:.0f}")
            if algorithmic and key in algorithmic:
                lines.append(f"{key}.algorithmic_bytes={algorithmic[key]}")
                lines.append(f"{key}.traffic_over_algorithmic={hbm / algorithmic[key]:.3f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the clock needs tens of milliseconds of load to settle")
    ap.add_argument("--only-main", action="store_true", help="skip secondary measurements and the CPU baseline")
    ap.add_argument("--only", default=None, choices=SECONDARY_NAMES,
                    help="run the main step and one secondary measurement only (for profiler passes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--gemv-iters", type=int, default=200)
    ap.add_argument("--side-iters", type=int, default=10)
    ap.add_argument("--summarize-pmc", metavar="OUT", help="write a counter summary from rocprofv3 CSV directories")
    ap.add_argument("--summarize-trace", metavar="OUT", help="write a kernel-trace summary from rocprofv3 CSV dirs")
    ap.add_argument("--dirs", nargs="*", default=[], help="rocprofv3 output directories (with --summarize-*)")
    ap.add_argument("--title", default="", help="summary title (with --summarize-*)")
    ap.add_argument("--command", nargs="*", default=[], help="the commands that made the CSVs (--summarize-*)")
    ap.add_argument("--sources", nargs="*", default=[], help="kernel sources hashed into the summary")
    ap.add_argument("--algorithmic", nargs="*", default=[], help="KERNEL@GRID=BYTES algorithmic bytes per launch")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.summarize_pmc:
        alg = dict(a.rsplit("=", 1) for a in args.algorithmic)
        summarize_pmc(args.dirs, args.summarize_pmc, args.title, args.command, args.sources,
                      {k: int(v) for k, v in alg.items()})
        return
    if args.summarize_trace:
        summarize_trace(args.dirs, args.summarize_trace, args.title, args.command)
        return
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
        for name in SECONDARY_NAMES:
            if args.only and name != args.only:
                continue
            fn, key = SECONDARY[name]
            log(f"secondary: {name}")
            sec[key] = fn(args, torch, mx, W)
            torch.cuda.empty_cache()
        if "ceilings" in sec and "w4a16_gemv_8192x8192" in sec:
            c = sec["ceilings"]["read_35.7MB_GB/s"]
            for M in W.GEMV_M:
                g = sec["w4a16_gemv_8192x8192"][f"M={M}"]
                g["frac_read_ceiling"] = g["GB/s"] / c
        out["secondary"] = sec
        if not args.no_cpu and not args.only:
            log("cpu baseline (oracle)")
            out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
