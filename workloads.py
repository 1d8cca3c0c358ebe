"""Seeded synthetic inputs for the five workloads (shapes of 70B-class layers).

This module only draws random numbers; it holds none of the quantization
arithmetic, so both the library's tests/bench and the CPU oracle use it.

Recipe (one independent PCG64 stream per tensor, seed 0):
  rng = numpy.random.default_rng([0, tensor_id]);  W = 1, X = 2, routing
  counts = 3, outlier columns = 4, outlier multipliers = 5.
  * weights      ~ N(0, 0.02) fp32
  * activations  ~ N(0, 1) fp32, with max(1, round(0.001 K)) distinct outlier
    columns multiplied (in fp32) by U[20, 100] -- or exactly 50 where the
    workload says x50 -- then RNE-cast to bf16 where the workload is bf16.
The pages place activation outliers in "<0.1%" of channels at "20x to 100x"
("NVFP4 Architecture", section "1. The Catastrophic Impact of Coarse-Grained
4-Bit Quantization").  Real model weights and datasets are not used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

W_ID, X_ID, COUNTS_ID, OUTLIER_COL_ID, OUTLIER_MUL_ID, ROUTER_ID = 1, 2, 3, 4, 5, 6


def _rng(tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id])


def normal(shape, sigma: float, tensor_id: int, seed: int = 0) -> np.ndarray:
    out = _rng(tensor_id, seed).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def n_outliers(K: int) -> int:
    return max(1, int(round(0.001 * K)))


def activations(M: int, K: int, outlier_mult="uniform", seed: int = 0) -> np.ndarray:
    """N(0,1) [M, K] fp32 with outlier columns scaled; outlier_mult is
    "uniform" (U[20, 100] per column) or a fixed number (e.g. 50.0)."""
    x = normal((M, K), 1.0, X_ID, seed)
    n = n_outliers(K)
    cols = _rng(OUTLIER_COL_ID, seed).choice(K, size=n, replace=False)
    if outlier_mult == "uniform":
        mult = _rng(OUTLIER_MUL_ID, seed).uniform(20.0, 100.0, size=n).astype(np.float32)
    else:
        mult = np.full(n, outlier_mult, dtype=np.float32)
    x[:, cols] *= mult[None, :]
    return x


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """RNE cast to bf16 (torch's CPU cast), returned as exact fp32 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def weights(N: int, K: int, sigma: float = 0.02, seed: int = 0) -> np.ndarray:
    return normal((N, K), sigma, W_ID, seed)


def expert_offsets(tokens: int, experts: int, seed: int = 0) -> np.ndarray:
    """Per-expert counts ~ Multinomial(tokens, uniform 1/experts); rows are
    pre-sorted by expert, offsets = prefix sums (int32, experts + 1)."""
    counts = _rng(COUNTS_ID, seed).multinomial(tokens, [1.0 / experts] * experts)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def topk_routing(tokens: int, experts: int, topk: int, seed: int = 0):
    """Top-k routing of a seeded router: logits ~ N(0, 1) [tokens, experts]
    (tensor id 6); each token takes its topk largest logits (distinct
    experts, largest first) with weights softmax over those topk logits.
    Returns (ids int32 [tokens, topk], weights fp32 [tokens, topk])."""
    logits = _rng(ROUTER_ID, seed).standard_normal(size=(tokens, experts), dtype=np.float32)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    top = np.take_along_axis(logits, ids.astype(np.int64), axis=1).astype(np.float64)
    e = np.exp(top - top.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    fmt: str          # "mxfp4" | "nvfp4"
    x_dtype: str      # "f32" | "bf16"
    out_dtype: str    # "f32" | "bf16"
    outlier: object   # "uniform" | float
    experts: int = 0
    w_sigma: float = 0.02


# The five workloads (sizes as named by the benchmark configurations).
C1 = Workload("mxfp4_quant_gemm_64x256x256", 64, 256, 256, "mxfp4", "f32", "f32", 50.0, w_sigma=1.0)
C2 = Workload("w4a16_gemv_M{1,8,16}_8192x8192", 16, 8192, 8192, "mxfp4", "bf16", "bf16", "uniform")
C3 = Workload("mxfp4_w4a4_gemm_4096x8192x8192", 4096, 8192, 8192, "mxfp4", "f32", "bf16", "uniform")
C4 = Workload("nvfp4_quant_w4a4_gemm_2048x28672x8192", 2048, 28672, 8192, "nvfp4", "f32", "bf16", 50.0)
C5 = Workload("moe_dynquant_grouped_gemm_8x4096x14336_T8192", 8192, 4096, 14336, "mxfp4", "bf16", "bf16",
              "uniform", experts=8)
GEMV_M = (1, 8, 16)
# Routed expert layer around C5's grouped product: 4096 tokens, top-2 of 8
# experts (8192 routed rows, the size of C5), same expert shapes.
MOE = Workload("moe_top2_route_quant_grouped_combine_8x4096x14336_T4096", 4096, 4096, 14336, "mxfp4", "bf16",
               "bf16", "uniform", experts=8)
MOE_TOPK = 2
# Wider MX elements on C3's product shape: activations and weights in
# (A format, B format) pairs -- FP8 activations with FP4 weights (W4A8), FP8 x
# FP8 and FP6 x FP6 -- from the same activation and weight recipes.
WIDE = Workload("mx_wide_gemm_4096x8192x8192", 4096, 8192, 8192, "mxfp8_e4m3", "bf16", "bf16", "uniform")
WIDE_PAIRS = (("mxfp8_e4m3", "mxfp4"), ("mxfp8_e4m3", "mxfp8_e4m3"), ("mxfp6_e2m3", "mxfp6_e2m3"))


def make(w: Workload, seed: int = 0, rows: int | None = None):
    """Inputs of workload w: returns dict with 'x' (fp32 values; bf16-exact
    when x_dtype is bf16), 'w' (fp32 weights, [E, N, K] when grouped) and
    'offsets' for the grouped workload.  rows limits the activation rows (a
    seeded prefix of the full tensor, for bounded CPU samples)."""
    M = w.M if rows is None else min(rows, w.M)
    x_full = activations(w.M, w.K, w.outlier, seed)
    x = x_full[:M]
    if w.x_dtype == "bf16":
        x = to_bf16_values(x)
    out = {"x": np.ascontiguousarray(x)}
    if w.experts:
        out["w"] = normal((w.experts, w.N, w.K), w.w_sigma, W_ID, seed)
        out["offsets"] = expert_offsets(w.M, w.experts, seed)
    else:
        out["w"] = weights(w.N, w.K, w.w_sigma, seed)
    return out
