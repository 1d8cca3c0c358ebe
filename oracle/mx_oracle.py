"""Plain fp64 oracle for MXFP4 / NVFP4 quantization, dequantization, GEMM, GEMV
and the grouped (MoE) GEMM with dynamic activation quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library.  Every step follows the pages' definitions in their order; readings of
points the pages leave open are marked READING.

Conventions shared with the library's public format (a format, not code):
  * a quantized tensor [R, K] has its blocks contiguous along K;
  * codes are packed two per byte, element 2j in the low nibble of byte j;
  * MXFP4 scale bytes are E8M0, NVFP4 scale bytes are FP8 E4M3, both [R, K/k].
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "E2M1_POSITIVE", "MX_BLOCK", "NV_BLOCK", "E4M3_MAX", "NV_GLOBAL_DIVISOR",
    "e2m1_value_from_bits", "e2m1_decode", "nearest_state_index",
    "e8m0_decode", "e4m3_value_from_bits", "e4m3_decode", "e4m3_nearest_code",
    "mx_block_exponent", "mxfp4_quantize", "nvfp4_global_scale",
    "nvfp4_quantize", "pack_codes", "unpack_codes", "dequantize",
    "round_to_bf16", "gemm", "gemm_tolerance", "gemv", "grouped_gemm",
    "naive_per_tensor_fp4", "storage_bytes", "moe_route", "moe_combine", "moe_forward", "rmsnorm_values", "rmsnorm_quantize", "rmsnorm_fragile", "MX_ELEMENT_FORMATS", "element_bits", "element_positive_values", "element_nearest_code", "mx_block_exponent_fmt", "pack_elements", "unpack_elements", "mx_quantize_fmt", "dequantize_fmt", "mx_quantize_variant", "dequantize_variant", "naive_per_tensor_quantize", "dequantize_naive", "reconstruction_snr_db",
]

# Table "The Complete Discrete State Mapping of E2M1" ("NVFP4 Architecture",
# section "1. The E2M1 Floating-Point Format"): the eight non-negative states.
E2M1_POSITIVE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

# Block lengths: 32 for MXFP4 ("How Microscaling FP4 (MXFP4) Halves Memory
# Bandwidth", section "The Microscaling Breakthrough: 32-Element Blocks"; the
# "MXFP4" wiki card, Core Facts) and 16 for NVFP4 ("NVIDIA NVFP4 quantization",
# section "The Physics of NVFP4").
MX_BLOCK = 32
NV_BLOCK = 16

# Largest finite FP8 E4M3 ("fn" variant, OCP FP8) value; NVFP4 block scales are
# E4M3 and the per-tensor scale maps the tensor maximum onto 6 * 448.
E4M3_MAX = 448.0
NV_GLOBAL_DIVISOR = 6.0 * E4M3_MAX  # READING: g = amax_tensor / (6 * 448)


# ---------------------------------------------------------------------------
# E2M1 element codec
# ---------------------------------------------------------------------------
def e2m1_value_from_bits(code: int) -> float:
    """Decode one 4-bit code from its bit fields ("NVFP4 Architecture", section
    "1. The E2M1 Floating-Point Format"): 1 sign bit, 2 exponent bits, 1
    mantissa bit; exponent field 0 is subnormal (0.5 * m), otherwise the value
    is 2^(e - 1) * (1 + m/2), i.e. exponent bias 1.  Zero is signed."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of unpacked 4-bit codes to float64 (table lookup,
    sign from bit 3; code 8 decodes to -0.0)."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = np.asarray(E2M1_POSITIVE, dtype=np.float64)[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


def nearest_state_index(mag: np.ndarray, unit: np.ndarray) -> np.ndarray:
    """Index i in 0..7 of the E2M1 state T[i] nearest to mag / unit.

    Equation q_i ("NVFP4 Architecture", section "1. The Dual-Level Mathematical
    Formulation"): each element maps to the nearest discrete E2M1 state after
    division by the scale; states beyond 6 do not exist, so larger values take
    6 (saturation, "How Microscaling FP4 (MXFP4)...", section "The
    Representation Dilemma: E2M1 vs. E3M0").
    READING: a value exactly half-way between two states goes to the state
    whose code is even (mantissa bit 0), i.e. round-to-nearest-even.

    The comparison is done in the scaled domain, |mag - T[i] * unit|, which
    orders the candidates exactly as |mag/unit - T[i]| does for unit > 0.
    Exactness in fp64: mag is an fp32 value (24 significant bits) and
    T[i] * unit has at most 2 + 24 + 4 significant bits, so every distance that
    can decide a near-tie is computed without rounding; distances that do
    round are separated by far more than their error.  unit == 0 (an NVFP4
    block whose scale rounded to zero) makes all candidates tie and gives 0.
    """
    mag = np.asarray(mag, dtype=np.float64)
    unit = np.asarray(unit, dtype=np.float64)
    cand = np.asarray(E2M1_POSITIVE, dtype=np.float64) * unit[..., None]
    dist = np.abs(mag[..., None] - cand)
    idx = np.argmin(dist, axis=-1)  # lowest index among equal minima
    # Half-way case: the tie partner is idx + 1; prefer the even code.
    nxt = np.minimum(idx + 1, 7)
    d_idx = np.take_along_axis(dist, idx[..., None], axis=-1)[..., 0]
    d_nxt = np.take_along_axis(dist, nxt[..., None], axis=-1)[..., 0]
    move = ((idx & 1) == 1) & (nxt != idx) & (d_nxt == d_idx)
    return (idx + move).astype(np.int64)


# ---------------------------------------------------------------------------
# Scale codecs
# ---------------------------------------------------------------------------
def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """E8M0 ("NVFP4 Architecture", section "2. Micro-Block Exponent Scaling:
    E8M0 Format"): unsigned 8-bit pure exponent with bias 127,
    S = 2^(E - 127).  (Byte 255 is NaN in OCP MX and is never produced.)"""
    return np.exp2(np.asarray(e, dtype=np.float64) - 127.0)


def e4m3_value_from_bits(b: int) -> float:
    """FP8 E4M3 ("fn": no infinities, 0x7F/0xFF are NaN) from its fields:
    sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal m/8 * 2^-6.  The NVFP4 block scale is E4M3 (the NVFP4 workload
    names it; the pages only say "8-bit")."""
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


_E4M3_POS = np.array([e4m3_value_from_bits(b) for b in range(0x7F)], dtype=np.float64)


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    table = np.array([e4m3_value_from_bits(i) for i in range(256)], dtype=np.float64)
    return table[b]


def e4m3_nearest_code(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Non-negative E4M3 code nearest to num / den (den > 0), ties to the even
    code, values past 448 saturating to 448 (code 0x7E).

    Compared in the scaled domain |num - c * den| over all 127 finite
    non-negative codes; c * den is exact in fp64 for den with <= 26 significant
    bits (den = 6 * g below), num is an fp32 value."""
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    dist = np.abs(num[..., None] - _E4M3_POS * den[..., None])
    idx = np.argmin(dist, axis=-1)
    nxt = np.minimum(idx + 1, 0x7E)
    d_idx = np.take_along_axis(dist, idx[..., None], axis=-1)[..., 0]
    d_nxt = np.take_along_axis(dist, nxt[..., None], axis=-1)[..., 0]
    move = ((idx & 1) == 1) & (nxt != idx) & (d_nxt == d_idx)
    return (idx + move).astype(np.uint8)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------
def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[R, K] 4-bit codes -> [R, K/2] bytes; element 2j in the low nibble.
    READING: the pages only say 16 codes occupy 64 bits ("NVFP4 Architecture",
    figure "OCP Microscaling (MXFP4 / NVFP4) Structural Decomposition"); the
    nibble order is our choice."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def storage_bytes(rows: int, cols: int, fmt: str) -> int:
    """Bytes of a quantized [rows, cols] tensor: 4-bit codes, one scale byte
    per block and, for NVFP4, one fp32 per-tensor scale."""
    k = MX_BLOCK if fmt == "mxfp4" else NV_BLOCK
    extra = 4 if fmt == "nvfp4" else 0
    return rows * cols // 2 + rows * cols // k + extra


# ---------------------------------------------------------------------------
# MXFP4
# ---------------------------------------------------------------------------
def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Block exponent e of S_block = 2^e.

    Equation S_block ("NVFP4 Architecture", section "1. The Dual-Level
    Mathematical Formulation"): S = 2^ceil(log2(max|x| / (6 * S_global))),
    with S_global = 1 for MXFP4 (READING: the pages' emulation has no global
    scale, and the MXFP4 workloads name none).  The emulation's guard
    max|x| >= 1e-8 ("End-to-End Implementation", step 1) is applied first.
    READING: ceil(log2(.)) is evaluated exactly -- e is the smallest integer
    with m <= 6 * 2^e -- not through a rounded floating-point log2.
    """
    m = np.maximum(np.asarray(amax, dtype=np.float64), float(np.float32(1e-8)))
    e = np.ceil(np.log2(m / 6.0)).astype(np.int64)  # estimate, then made exact
    for _ in range(2):
        e = np.where(6.0 * np.exp2(e.astype(np.float64)) < m, e + 1, e)
        e = np.where(6.0 * np.exp2((e - 1).astype(np.float64)) >= m, e - 1, e)
    return e


def mxfp4_quantize(x: np.ndarray, block: int = MX_BLOCK):
    """MXFP4 quantization of a row-major [R, K] fp32 tensor, K % 32 == 0.

    Steps of the pages' emulation ("End-to-End Implementation: Emulating NVFP4
    & Microscaling in PyTorch"): view as blocks, block max |x|, power-of-two
    scale, divide, nearest E2M1 state with the input's sign.  Block length 32
    (MXFP4); block=16 gives the 16-element E8M0 variant the emulation uses by
    default.  Returns (packed codes uint8 [R, K/2], E8M0 scale bytes uint8
    [R, K/block]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the block length")
    xb = x.astype(np.float64).reshape(R, K // block, block)
    amax = np.abs(xb).max(axis=-1)
    e = mx_block_exponent(amax)
    unit = np.exp2(e.astype(np.float64))  # S_block (S_global = 1)
    sign = np.signbit(x).reshape(xb.shape).astype(np.int64)  # READING: copy the sign, also of 0
    codes = np.empty(xb.shape, dtype=np.uint8)
    step = max(1, (1 << 22) // max(K, 1))  # rows per chunk: bounds the distance arrays
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        idx = nearest_state_index(np.abs(xb[r0:r1]),
                                  np.broadcast_to(unit[r0:r1, :, None], xb[r0:r1].shape))
        codes[r0:r1] = (idx | (sign[r0:r1] << 3)).astype(np.uint8)
    return pack_codes(codes.reshape(R, K)), (e + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# NVFP4
# ---------------------------------------------------------------------------
def nvfp4_global_scale(x: np.ndarray) -> np.float32:
    """Per-tensor scale S_global ("NVFP4 Architecture", section "1. The
    Dual-Level Mathematical Formulation": the tensor's dynamic ceiling).
    READING (parity unpinned): g = fp32(max|x| / (6 * 448)) correctly rounded,
    so that the largest block scale is E4M3's maximum 448; g = 1 when x == 0."""
    a = np.float32(np.abs(np.asarray(x, dtype=np.float32)).max()) if np.asarray(x).size else np.float32(0)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a) / np.float32(NV_GLOBAL_DIVISOR)  # IEEE fp32 division


def nvfp4_quantize(x: np.ndarray, global_scale=None):
    """NVFP4 quantization of a row-major [R, K] fp32 tensor, K % 16 == 0.

    Dual-level scaling ("NVFP4 Architecture", section "1. The Dual-Level
    Mathematical Formulation") with 16-element blocks ("NVIDIA NVFP4
    quantization", section "The Physics of NVFP4") and an E4M3 block scale:
      g      = per-tensor scale (nvfp4_global_scale, or the given static one)
      s_b    = E4M3 nearest to max_b|x| / (6 g)  (block scale = amax / 6)
      q_i    = E2M1 nearest to x_i / (s_b g), saturating at +-6
    Returns (packed codes [R, K/2], E4M3 bytes [R, K/16], g as np.float32).
    """
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    g = nvfp4_global_scale(x) if global_scale is None else np.float32(global_scale)
    g64 = np.float64(g)
    xb = x.astype(np.float64).reshape(R, K // NV_BLOCK, NV_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    sbytes = np.empty(amax.shape, dtype=np.uint8)
    codes = np.empty(xb.shape, dtype=np.uint8)
    sign = np.signbit(x).reshape(xb.shape).astype(np.int64)
    step = 256  # rows per chunk: bounds the [rows, blocks, candidates] distance arrays
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        sb = e4m3_nearest_code(amax[r0:r1], np.full(amax[r0:r1].shape, 6.0 * g64))
        sbytes[r0:r1] = sb
        unit = _E4M3_POS[sb.astype(np.int64)] * g64  # s_b * g, exact in fp64
        idx = nearest_state_index(np.abs(xb[r0:r1]),
                                  np.broadcast_to(unit[..., None], xb[r0:r1].shape))
        codes[r0:r1] = (idx | (sign[r0:r1] << 3)).astype(np.uint8)
    return pack_codes(codes.reshape(R, K)), sbytes, np.float32(g)


# ---------------------------------------------------------------------------
# Dequantization
# ---------------------------------------------------------------------------
def dequantize(fmt: str, packed: np.ndarray, scales: np.ndarray, global_scale=None) -> np.ndarray:
    """Reconstruction x_hat = q * S_block * S_global ("NVFP4 Architecture",
    section "1. The Dual-Level Mathematical Formulation", equation x_hat).
    MXFP4: q * 2^(E-127), exact in fp32.  NVFP4: fp32(fp32(q * s_b) * g); the
    inner product is exact, the multiplication by g rounds once.
    Returns fp32 [R, K]."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    q = e2m1_decode(codes)
    if fmt == "mxfp4":
        s = np.repeat(e8m0_decode(scales), K // np.asarray(scales).shape[1], axis=1)
        return (q * s).astype(np.float32)
    if fmt == "nvfp4":
        s = np.repeat(e4m3_decode(scales), NV_BLOCK, axis=1)
        qs = (q * s).astype(np.float32)  # exact: <= 6 significant bits
        return (qs * np.float32(global_scale)).astype(np.float32)  # fp32 multiply
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# Products
# ---------------------------------------------------------------------------
def round_to_bf16(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, returned as the fp32 values of the
    bf16 results (finite inputs)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    b = y.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def gemm(a_hat: np.ndarray, b_hat: np.ndarray, out: str = "f32") -> np.ndarray:
    """Y = X . W ("NVFP4 Architecture", section "1. The Dual-Level Mathematical
    Formulation") with X = a_hat [M, K] and W given as b_hat [N, K]
    (READING: both operands K-contiguous, C row-major [M, N]).
    Sum in fp64 (a library matmul), rounded once to fp32; out="bf16" rounds
    that fp32 to bf16 (nearest-even)."""
    y = np.matmul(np.asarray(a_hat, np.float64), np.asarray(b_hat, np.float64).T).astype(np.float32)
    return round_to_bf16(y) if out == "bf16" else y


def gemm_tolerance(a_hat: np.ndarray, b_hat: np.ndarray, y_ref: np.ndarray | None = None,
                   out: str = "f32", rel: float = 1e-5) -> np.ndarray:
    """Per-element bound rel * sum_k |a||b| on the dequantized operands.
    READING: a bf16 output adds one bf16 ulp of the reference value, since the
    final rounding alone can exceed the fp32 bound."""
    tol = rel * np.matmul(np.abs(np.asarray(a_hat, np.float64)), np.abs(np.asarray(b_hat, np.float64)).T)
    if out == "bf16":
        assert y_ref is not None
        mag = np.abs(np.asarray(y_ref, np.float64))
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
        ulp = np.where(mag > 0, np.exp2(e - 7), 2.0 ** -133)
        tol = tol + ulp
    return tol


def gemv(x_bf16_values: np.ndarray, w_packed, w_scales, fmt: str = "mxfp4", w_global=None) -> np.ndarray:
    """W4A16: y = x . W_hat^T with bf16 activations (exact in fp32) and the
    dequantized 4-bit weights ("Extreme Quantization and Precision
    Engineering", section "Key points": weights compressed, math in 16-bit).
    Returns bf16 values as fp32 [M, N]."""
    w_hat = dequantize(fmt, w_packed, w_scales, w_global)
    return gemm(np.asarray(x_bf16_values, np.float32), w_hat, out="bf16")


def grouped_gemm(x: np.ndarray, offsets: np.ndarray, w_packed: np.ndarray, w_scales: np.ndarray):
    """Grouped (mixture-of-experts) product with dynamic activation
    quantization: for every expert g and rows r in [off[g], off[g+1]),
    Y[r] = MXFP4(X[r]) . W_hat_g^T, bf16 output.  Activations are quantized per
    layer at run time ("How Microscaling FP4 (MXFP4)...", section "Native
    Pre-Training vs. Post-Training Quantization"); routed experts are where
    the pages place the largest gain ("NVFP4 Architecture", section
    "Strategic Recommendations").
    x: fp32 values [T, K]; w_packed [G, N, K/2]; w_scales [G, N, K/32].
    Returns (Y bf16-as-fp32 [T, N], activation codes [T, K/2], scales [T, K/32])."""
    x = np.asarray(x, np.float32)
    G = w_packed.shape[0]
    N = w_packed.shape[1]
    T, K = x.shape
    y = np.zeros((T, N), np.float32)
    a_codes, a_scales = mxfp4_quantize(x) if T else (np.zeros((0, K // 2), np.uint8), np.zeros((0, K // 32), np.uint8))
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        a_hat = dequantize("mxfp4", a_codes[r0:r1], a_scales[r0:r1])
        w_hat = dequantize("mxfp4", w_packed[g], w_scales[g])
        y[r0:r1] = gemm(a_hat, w_hat, out="bf16")
    return y, a_codes, a_scales


# ---------------------------------------------------------------------------
# The wider members of the MX family: MXFP8 (E4M3, E5M2) and MXFP6 (E2M3,
# E3M2) elements with the same 32-element blocks and E8M0 scales ("MXFP4"
# card, section "Core Facts": MXFP8/MXFP4 scaled GEMM; "How Microscaling FP4
# (MXFP4)...", section "The Representation Dilemma: E2M1 vs. E3M0" for the
# element/exponent trade-off).  Reading: the pages' scale rule carries over
# with the format's largest finite value Emax in place of 6 -- e is the
# smallest integer with amax <= Emax * 2^e (amax >= fp32(1e-8) as in the
# emulation) -- and elements round to nearest, ties to the even code.
# ---------------------------------------------------------------------------
MX_ELEMENT_FORMATS = {
    # name: (exponent bits, mantissa bits, bias, largest finite value)
    "mxfp8_e4m3": (4, 3, 7, 448.0),
    "mxfp8_e5m2": (5, 2, 15, 57344.0),
    "mxfp6_e2m3": (2, 3, 1, 7.5),
    "mxfp6_e3m2": (3, 2, 3, 28.0),
    "mxfp4": (2, 1, 1, 6.0),
}


def element_bits(fmt: str) -> int:
    E, M, _, _ = MX_ELEMENT_FORMATS[fmt]
    return 1 + E + M


def element_positive_values(fmt: str) -> np.ndarray:
    """Values of the non-negative finite codes 0, 1, 2, ... of a minifloat
    (sign bit clear), from the fields: exponent field 0 is subnormal
    (m / 2^M * 2^(1-bias)), otherwise (1 + m / 2^M) * 2^(e - bias); codes
    above Emax (E4M3's NaN, E5M2's infinities and NaNs) are excluded."""
    E, M, bias, emax = MX_ELEMENT_FORMATS[fmt]
    vals = []
    for code in range(1 << (E + M)):
        e, m = code >> M, code & ((1 << M) - 1)
        v = (m / 2.0 ** M) * 2.0 ** (1 - bias) if e == 0 else (1 + m / 2.0 ** M) * 2.0 ** (e - bias)
        if v > emax:
            break
        vals.append(v)
    return np.array(vals, np.float64)


def element_nearest_code(v: np.ndarray, fmt: str) -> np.ndarray:
    """Code of the non-negative value nearest to v >= 0 (exact fp64 inputs),
    ties to the even code, v above Emax saturating to Emax."""
    table = element_positive_values(fmt)
    v = np.asarray(v, np.float64)
    d = np.abs(v[..., None] - table)
    idx = np.argmin(d, axis=-1)
    tie = (idx % 2 == 1) & (idx + 1 < len(table))
    nxt = np.minimum(idx + 1, len(table) - 1)
    tie &= np.take_along_axis(d, nxt[..., None], -1)[..., 0] == np.take_along_axis(d, idx[..., None], -1)[..., 0]
    return np.where(tie, nxt, idx).astype(np.int64)


def mx_block_exponent_fmt(amax: np.ndarray, fmt: str) -> np.ndarray:
    """Smallest integer e with amax <= Emax * 2^e, amax first raised to
    fp32(1e-8); exact (a correction loop around the fp64 log2 estimate)."""
    emax = MX_ELEMENT_FORMATS[fmt][3]
    a = np.maximum(np.asarray(amax, np.float64), float(np.float32(1e-8)))
    e = np.ceil(np.log2(a / emax)).astype(np.int64)
    e = np.where(emax * np.exp2(e.astype(np.float64)) < a, e + 1, e)
    e = np.where(emax * np.exp2((e - 1).astype(np.float64)) >= a, e - 1, e)
    return e


def pack_elements(codes: np.ndarray, bits: int) -> np.ndarray:
    """[R, K] codes of `bits` bits -> [R, K*bits/8] bytes, element i at bits
    [bits*i, bits*i + bits) of the row's little-endian bit stream."""
    codes = np.asarray(codes, np.uint64)
    R, K = codes.shape
    if bits == 8:
        return codes.astype(np.uint8)
    if bits == 4:
        return pack_codes(codes.astype(np.uint8))
    assert bits == 6 and K % 4 == 0
    g = codes.reshape(R, K // 4, 4)
    word = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    out = np.stack([(word >> (8 * b)) & 0xFF for b in range(3)], axis=-1)
    return out.reshape(R, K * 3 // 4).astype(np.uint8)


def unpack_elements(packed: np.ndarray, bits: int) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    R = packed.shape[0]
    if bits == 8:
        return packed.astype(np.int64)
    if bits == 4:
        return unpack_codes(packed).astype(np.int64)
    g = packed.reshape(R, -1, 3).astype(np.uint64)
    word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    out = np.stack([(word >> (6 * i)) & 0x3F for i in range(4)], axis=-1)
    return out.reshape(R, -1).astype(np.int64)


def mx_quantize_fmt(x: np.ndarray, fmt: str):
    """MX quantization of a row-major [R, K] fp32 tensor (K % 32 == 0) with
    elements of `fmt`: per 32-element block the E8M0 byte e + 127 and each
    element the code nearest to x / 2^e (sign bit = x's sign).
    Returns (packed codes [R, K*bits/8], scale bytes [R, K/32])."""
    x = np.asarray(x, np.float32)
    R, K = x.shape
    bits = element_bits(fmt)
    xb = x.reshape(R, K // 32, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=-1)
    e = mx_block_exponent_fmt(amax, fmt)
    mag = np.abs(xb) * np.exp2(-e.astype(np.float64))[..., None]
    idx = element_nearest_code(mag, fmt)
    sign = np.signbit(x.reshape(R, K // 32, 32)).astype(np.int64)
    codes = idx | (sign << (bits - 1))
    return pack_elements(codes.reshape(R, K), bits), (e + 127).astype(np.uint8)


def dequantize_fmt(fmt: str, packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_hat = value(code) * 2^(E - 127) for the MX element formats (exact in
    fp32 for every format and scale the quantizer emits)."""
    bits = element_bits(fmt)
    codes = unpack_elements(packed, bits)
    R, K = codes.shape
    E, M, bias, _ = MX_ELEMENT_FORMATS[fmt]
    mag_code = codes & ((1 << (bits - 1)) - 1)
    e, m = mag_code >> M, mag_code & ((1 << M) - 1)
    mag = np.where(e == 0, m / 2.0 ** M * 2.0 ** (1 - bias), (1 + m / 2.0 ** M) * np.exp2((e - bias).astype(np.float64)))
    val = np.where((codes >> (bits - 1)) & 1, -mag, mag)
    s = np.exp2(np.asarray(scales, np.float64) - 127.0)
    return (val.reshape(R, K // 32, 32) * s[..., None]).reshape(R, K).astype(np.float32)


# ---------------------------------------------------------------------------
# Variants of the pages' emulation surface ("NVFP4 Architecture", sections
# "1. The Dual-Level Mathematical Formulation" and "End-to-End
# Implementation"): any block length (the emulation defaults to 16 with an
# E8M0 scale), an optional per-tensor scale S_global inside the power-of-two
# block scale, the OCP floor rule as an alternative exponent rule, and rows
# whose length is not a multiple of the block (zero-padded, as the emulation
# pads its flattened tensor).
# ---------------------------------------------------------------------------
def _emax_exponent(fmt: str) -> int:
    """floor(log2 Emax): 2 for E2M1 and E2M3, 8 for E4M3, 15 for E5M2, 4 for E3M2."""
    return int(math.floor(math.log2(MX_ELEMENT_FORMATS[fmt][3])))


def mx_quantize_variant(x: np.ndarray, fmt: str = "mxfp4", block: int = 32, rule: str = "ceil",
                        global_scale=None):
    """Block quantization with E8M0 scales, generalised.

    Rows are zero-padded to Kp = ceil(K / block) * block (READING: blocks stay
    inside a row, the emulation's zero padding applied per row; the padding
    leaves max|x| unchanged and its codes are +0).  With g = global_scale
    (fp32; 1 when None) and Emax the element format's largest value:
      rule "ceil"  (the pages): e = smallest integer with max(m, 1e-8) <= Emax * g * 2^e;
      rule "floor" (OCP, READING: offered as an option only, g must be 1):
                   e = floor(log2 max(m, 1e-8)) - floor(log2 Emax); elements
                   beyond Emax then saturate to +-Emax.
    Elements: the code nearest to x / (g * 2^e) (ties to the even code), the
    input's sign kept.  Returns (packed codes [R, Kp * bits / 8], E8M0 bytes
    [R, Kp / block])."""
    x = np.asarray(x, np.float32)
    R, K = x.shape
    Kp = -(-K // block) * block
    xp = np.zeros((R, Kp), np.float32)
    xp[:, :K] = x
    g = 1.0 if global_scale is None else float(np.float32(global_scale))
    bits = element_bits(fmt)
    emax = MX_ELEMENT_FORMATS[fmt][3]
    xb = xp.astype(np.float64).reshape(R, Kp // block, block)
    m = np.maximum(np.abs(xb).max(axis=-1), float(np.float32(1e-8)))
    if rule == "ceil":
        lim = emax * g
        e = np.ceil(np.log2(m / lim)).astype(np.int64)
        for _ in range(2):   # exact: products of Emax, g and 2^e are exact in fp64
            e = np.where(lim * np.exp2(e.astype(np.float64)) < m, e + 1, e)
            e = np.where(lim * np.exp2((e - 1).astype(np.float64)) >= m, e - 1, e)
    elif rule == "floor":
        if g != 1.0:
            raise ValueError("the floor rule has no per-tensor scale")
        e = np.floor(np.log2(m)).astype(np.int64)
        e = np.where(np.exp2(e.astype(np.float64)) > m, e - 1, e)
        e = np.where(np.exp2((e + 1).astype(np.float64)) <= m, e + 1, e)
        e = e - _emax_exponent(fmt)
    else:
        raise ValueError(rule)
    unit = g * np.exp2(e.astype(np.float64))
    # nearest code: compare |x| with the exact midpoints between codes times
    # the unit (fp64 products of an fp32 g, a power of two and a short midpoint)
    table = element_positive_values(fmt)
    mids = (table[:-1] + table[1:]) / 2
    above = np.abs(xb)[..., None] > mids * unit[..., None, None]
    at = np.abs(xb)[..., None] == mids * unit[..., None, None]
    idx = above.sum(-1) + (at & (np.arange(len(mids)) % 2 == 1)).sum(-1)   # ties go to the even code
    sign = np.signbit(xp).reshape(xb.shape).astype(np.int64)
    codes = idx.astype(np.int64) | (sign << (bits - 1))
    return pack_elements(codes.reshape(R, Kp), bits), (e + 127).astype(np.uint8)


def dequantize_variant(fmt: str, packed: np.ndarray, scales: np.ndarray, K: int, global_scale=None) -> np.ndarray:
    """x_hat = fp32(fp32(value(code) * 2^(E-127)) * g) for the first K columns."""
    y = dequantize_fmt(fmt, packed, scales) if fmt != "mxfp4" else None
    if fmt == "mxfp4":
        codes = unpack_codes(packed)
        R, Kp = codes.shape
        s = np.repeat(e8m0_decode(scales), Kp // np.asarray(scales).shape[1], axis=1)
        y = (e2m1_decode(codes) * s).astype(np.float32)
    if global_scale is not None:
        y = (y * np.float32(global_scale)).astype(np.float32)
    return y[:, :K]


def naive_per_tensor_quantize(x: np.ndarray):
    """The pages' naive per-tensor FP4 in stored form: one fp32 scale
    s = fp32(max(max|x|, 1e-8) / 6) for the whole tensor (READING: the
    emulation computes it in the tensor's fp32), every element the E2M1 state
    nearest to x / s with the input's sign.  Returns (packed codes [R, K/2]
    (K even), s as np.float32)."""
    x = np.asarray(x, np.float32)
    s = np.float32(max(np.float32(np.abs(x).max()) if x.size else np.float32(0), np.float32(1e-8))) / np.float32(6.0)
    idx = nearest_state_index(np.abs(x.astype(np.float64)), np.full(x.shape, float(s)))
    codes = (idx | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)
    return pack_codes(codes), np.float32(s)


def dequantize_naive(packed: np.ndarray, s) -> np.ndarray:
    return (e2m1_decode(unpack_codes(packed)) * np.float64(np.float32(s))).astype(np.float32)


def reconstruction_snr_db(x: np.ndarray, x_hat: np.ndarray) -> float:
    """10 log10(sum x^2 / sum (x - x_hat)^2) in fp64: the accuracy measure of
    the pages' emulation demo (MSE against the original, reported as SNR)."""
    x = np.asarray(x, np.float64)
    d = x - np.asarray(x_hat, np.float64)
    num, den = float(np.sum(x * x)), float(np.sum(d * d))
    return float("inf") if den == 0 else 10.0 * math.log10(num / den)


def moe_route(topk_ids: np.ndarray, experts: int):
    """Expert-sorted order of top-k routed (token, slot) pairs.  Routed expert
    layers are where block-scaled FP4 gains most ("NVFP4 Architecture", section
    "Strategic Recommendations: Adopting NVFP4 in 2026"; TopK and grouped GEMM
    in the "MXFP4" card, section "Core Facts").  Reading: a stable sort by
    expert id -- the pairs of one expert keep their flat order t * topk + s;
    pairs whose id is outside [0, experts) are dropped (row -1).
    Returns (offsets [experts+1], dest_row [T*topk], src_token [offsets[-1]])."""
    ids = np.asarray(topk_ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    dest = np.full(T * k, -1, np.int64)
    offsets = np.zeros(experts + 1, np.int64)
    src = []
    row = 0
    for g in range(experts):
        offsets[g] = row
        for p in range(T * k):          # flat order = stable
            if flat[p] == g:
                dest[p] = row
                src.append(p // k)
                row += 1
    offsets[experts] = row
    return offsets.astype(np.int32), dest.astype(np.int32), np.asarray(src, np.int32)


def moe_combine(y: np.ndarray, dest_row: np.ndarray, weights: np.ndarray, tokens: int, topk: int) -> np.ndarray:
    """out[t] = sum_s w[t, s] * y[dest_row[t, s]], summed in fp64 and rounded
    once to fp32; pairs with row -1 add nothing."""
    y = np.asarray(y, np.float64)
    w = np.asarray(weights, np.float64).reshape(tokens, topk)
    d = np.asarray(dest_row).reshape(tokens, topk)
    out = np.zeros((tokens, y.shape[1]), np.float64)
    for t in range(tokens):
        for s in range(topk):
            if 0 <= d[t, s] < y.shape[0]:
                out[t] += w[t, s] * y[d[t, s]]
    return out.astype(np.float32)


def moe_forward(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, w_packed: np.ndarray,
                w_scales: np.ndarray, y_out: str = "bf16", out: str = "bf16"):
    """A routed W4A4 expert layer: route, quantize each routed token's
    activations to MXFP4 (in sorted order), multiply by its expert's MXFP4
    weights (fp64 sums rounded to fp32, then to y_out), combine with the
    routing weights.  x fp32 values [T, K]; w_packed [G, N, K/2]; w_scales
    [G, N, K/32].  Returns (out [T, N], dict of the intermediates)."""
    x = np.asarray(x, np.float32)
    T, K = x.shape
    G, N = w_packed.shape[0], w_packed.shape[1]
    k = topk_ids.shape[1]
    offsets, dest, src = moe_route(topk_ids, G)
    xs = x[src] if len(src) else np.zeros((0, K), np.float32)
    y, a_codes, a_scales = grouped_gemm(xs, offsets, w_packed, w_scales)
    if y_out == "f32":
        y = np.zeros((len(src), N), np.float32)
        for g in range(G):
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            if r1 > r0:
                y[r0:r1] = gemm(dequantize("mxfp4", a_codes[r0:r1], a_scales[r0:r1]),
                                dequantize("mxfp4", w_packed[g], w_scales[g]), out="f32")
    o = moe_combine(y, dest, topk_w, T, k)
    if out == "bf16":
        o = round_to_bf16(o)
    return o, {"offsets": offsets, "dest_row": dest, "src_token": src, "y": y,
               "a_codes": a_codes, "a_scales": a_scales}


def rmsnorm_values(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm by its definition, in fp64: y = x / sqrt(mean(x^2) + eps) * gamma
    per row (RMSNorm appears on the pages only as an operation of an MXFP4
    serving stack, "MXFP4" card, section "Core Facts").  x and gamma are the
    fp32 values given (bf16 activations are exact in fp32), eps the value as
    passed (an fp32 number).  Returns float64 [R, K]: a kernel computing in
    fp32 lands within its own rounding error of these values."""
    x = np.asarray(x, np.float64)
    gamma = np.asarray(gamma, np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * gamma


def rmsnorm_quantize(x: np.ndarray, gamma: np.ndarray, eps: float, fmt: str = "mxfp4", global_scale=None):
    """Block quantization of the RMSNorm output (rmsnorm_values rounded to
    the nearest fp32): MXFP4, or NVFP4 with a given static per-tensor scale.
    Where an fp64 value lies within a kernel's fp32 error of a decision
    boundary the kernel's code may legitimately differ; the comparison
    excludes exactly those decisions (see rmsnorm_fragile)."""
    y = rmsnorm_values(x, gamma, eps).astype(np.float32)
    if fmt == "mxfp4":
        return mxfp4_quantize(y)
    c, s, _ = nvfp4_quantize(y, global_scale=global_scale)
    return c, s


def rmsnorm_fragile(y64: np.ndarray, rel: float, fmt: str = "mxfp4", global_scale=None):
    """Decisions of the quantization of y64 that a relative perturbation of at
    most `rel` of every value can change: (block mask [R, K/k], element mask
    [R, K]).  A block is fragile when its scale byte differs between
    max|y|(1 - rel) and max|y|(1 + rel); an element when its state differs
    between |y|(1 - rel) and |y|(1 + rel) at the block's scale."""
    y64 = np.asarray(y64, np.float64)
    R, K = y64.shape
    k = MX_BLOCK if fmt == "mxfp4" else NV_BLOCK
    mag = np.abs(y64).reshape(R, K // k, k)
    m = mag.max(axis=-1)
    lo, hi = 1.0 - rel, 1.0 + rel
    if fmt == "mxfp4":
        e_lo, e_hi = mx_block_exponent(m * lo), mx_block_exponent(m * hi)
        block = e_lo != e_hi
        unit = np.exp2(mx_block_exponent(m).astype(np.float64))
    else:
        g64 = float(np.float32(global_scale))
        den = np.full(m.shape, 6.0 * g64)
        s_lo, s_hi = e4m3_nearest_code(m * lo, den), e4m3_nearest_code(m * hi, den)
        block = s_lo != s_hi
        unit = _E4M3_POS[e4m3_nearest_code(m, den).astype(np.int64)] * g64
    u = np.broadcast_to(unit[..., None], mag.shape)
    elem = nearest_state_index(mag * lo, u) != nearest_state_index(mag * hi, u)
    return block, elem.reshape(R, K)


def naive_per_tensor_fp4(x: np.ndarray) -> np.ndarray:
    """The pages' coarse baseline ("End-to-End Implementation", function
    naive_per_tensor_fp4; figure "The Outlier Distortion in Coarse-Grained
    FP4"): one scale max|x| / 6 for the whole tensor (not a power of two),
    nearest E2M1 state, returned dequantized (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    s = max(float(np.abs(x).max()), 1e-8) / 6.0
    idx = nearest_state_index(np.abs(x) / s, np.ones(x.shape))
    q = np.asarray(E2M1_POSITIVE)[idx]
    return np.where(np.signbit(x), -q, q) * s
