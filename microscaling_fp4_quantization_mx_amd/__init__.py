"""Python binding of libmx (block-scaled FP4 quantization and GEMM on gfx950).

Argument marshalling only: every step runs in the HIP kernels of libmx.so.
PyTorch provides device memory and the current stream.  The functions carry
the C names (mx_quantize, mx_dequantize, mx_gemm, mx_gemv, ...); the raw
ctypes entry points are available as ``lib().mx_*``.

There is no fallback: if libmx.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "MXError", "MXTensor", "lib", "library_path", "MX_FMT_MXFP4", "MX_FMT_NVFP4", "MX_DT_F32", "MX_DT_BF16",
    "MX_QUANT_STATIC_GLOBAL", "MX_OP_QUANTIZE", "MX_OP_GEMM", "STATUS", "CMxTensor", "CMxGemmArgs",
    "empty_quantized", "mx_quantize", "mx_dequantize", "mx_gemm", "mx_gemv", "mx_workspace_bytes",
    "mx_status_string", "mx_version", "MX_OP_MOE_ROUTE", "mx_moe_route", "mx_quantize_rows", "mx_moe_combine",
    "moe_forward", "mx_rmsnorm_quantize", "MX_FMT_MXFP8_E4M3", "MX_FMT_MXFP8_E5M2", "MX_FMT_MXFP6_E2M3",
    "MX_FMT_MXFP6_E3M2", "element_bits", "MX_FMT_MXFP4_K16", "MX_FMT_FP4_TENSOR", "MX_QUANT_SCALE_FLOOR",
    "padded_cols", "mx_quantize_noalloc", "MX_GEMM_F8F6F4_MATRIX_CORES", "MX_GEMM_FUSED_QUANTIZE",
    "MX_GEMM_DYNAMIC_A_FORMAT",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmx.so")

MX_FMT_MXFP4, MX_FMT_NVFP4 = 0, 1
MX_FMT_MXFP8_E4M3, MX_FMT_MXFP8_E5M2, MX_FMT_MXFP6_E2M3, MX_FMT_MXFP6_E3M2 = 2, 3, 4, 5
MX_FMT_MXFP4_K16, MX_FMT_FP4_TENSOR = 6, 7
MX_DT_F32, MX_DT_BF16 = 0, 1
MX_QUANT_DEFAULT, MX_QUANT_STATIC_GLOBAL, MX_QUANT_SCALE_FLOOR = 0, 1, 2
MX_OP_QUANTIZE, MX_OP_GEMM, MX_OP_MOE_ROUTE = 0, 1, 2
MX_GEMM_F8F6F4_MATRIX_CORES, MX_GEMM_FUSED_QUANTIZE = 1, 2


def MX_GEMM_DYNAMIC_A_FORMAT(fmt: int) -> int:
    """mx_gemm flag bits naming the format a dynamic A is quantized to."""
    return (fmt + 1) << 4


STATUS = {0: "MX_OK", -1: "MX_ERR_NULL", -2: "MX_ERR_SHAPE", -3: "MX_ERR_ALIGN", -4: "MX_ERR_DTYPE",
          -5: "MX_ERR_UNSUPPORTED", -6: "MX_ERR_HIP", -7: "MX_ERR_WORKSPACE", -8: "MX_ERR_FORMAT"}
_FMT = {"mxfp4": MX_FMT_MXFP4, "nvfp4": MX_FMT_NVFP4, "mxfp8_e4m3": MX_FMT_MXFP8_E4M3,
        "mxfp8_e5m2": MX_FMT_MXFP8_E5M2, "mxfp6_e2m3": MX_FMT_MXFP6_E2M3, "mxfp6_e3m2": MX_FMT_MXFP6_E3M2,
        "mxfp4_k16": MX_FMT_MXFP4_K16, "fp4_tensor": MX_FMT_FP4_TENSOR}
_BLOCK = {MX_FMT_MXFP4: 32, MX_FMT_NVFP4: 16, MX_FMT_MXFP8_E4M3: 32, MX_FMT_MXFP8_E5M2: 32,
          MX_FMT_MXFP6_E2M3: 32, MX_FMT_MXFP6_E3M2: 32, MX_FMT_MXFP4_K16: 16, MX_FMT_FP4_TENSOR: 2}
_BITS = {MX_FMT_MXFP4: 4, MX_FMT_NVFP4: 4, MX_FMT_MXFP8_E4M3: 8, MX_FMT_MXFP8_E5M2: 8,
         MX_FMT_MXFP6_E2M3: 6, MX_FMT_MXFP6_E3M2: 6, MX_FMT_MXFP4_K16: 4, MX_FMT_FP4_TENSOR: 4}


def padded_cols(cols: int, fmt) -> int:
    """Stored row length: E8M0-scaled formats pad rows to whole blocks."""
    f = _FMT[fmt] if isinstance(fmt, str) else fmt
    k = _BLOCK[f]
    return -(-cols // k) * k if f not in (MX_FMT_NVFP4, MX_FMT_FP4_TENSOR) else cols


def element_bits(fmt) -> int:
    """Bits per element code of a format (name or MX_FMT_* value)."""
    return _BITS[_FMT[fmt] if isinstance(fmt, str) else fmt]


class MXError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)} ({mx_status_string(status)})")


class CMxTensor(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p)]


class CMxGemmArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a", ctypes.POINTER(CMxTensor)), ("a_raw", ctypes.c_void_p), ("a_raw_dtype", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("lda_raw", ctypes.c_int64), ("b", ctypes.POINTER(CMxTensor)),
                ("group_offsets", ctypes.c_void_p), ("c", ctypes.c_void_p), ("c_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("ldc", ctypes.c_int64), ("a_codes_out", ctypes.c_void_p),
                ("a_scales_out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libmx.so (built in-tree by build.py); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built: run `python -m microscaling_fp4_quantization_mx_amd.build`"
                               " (there is no CPU fallback)")
        L = ctypes.CDLL(library_path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.mx_quantize.argtypes = [vp, i32, i64, ctypes.POINTER(CMxTensor), i32, vp, sz, vp]
        L.mx_quantize.restype = ctypes.c_int
        L.mx_quantize_noalloc.argtypes = [vp, i32, i64, ctypes.POINTER(CMxTensor), i32, vp]
        L.mx_quantize_noalloc.restype = ctypes.c_int
        L.mx_dequantize.argtypes = [ctypes.POINTER(CMxTensor), vp, i32, i64, vp]
        L.mx_dequantize.restype = ctypes.c_int
        L.mx_gemm.argtypes = [ctypes.POINTER(CMxGemmArgs), vp]
        L.mx_gemm.restype = ctypes.c_int
        L.mx_gemv.argtypes = [vp, i32, i64, i64, ctypes.POINTER(CMxTensor), vp, i32, i64, vp]
        L.mx_gemv.restype = ctypes.c_int
        L.mx_moe_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, sz, vp]
        L.mx_moe_route.restype = ctypes.c_int
        L.mx_quantize_rows.argtypes = [vp, i32, i64, i64, vp, ctypes.POINTER(CMxTensor), vp]
        L.mx_quantize_rows.restype = ctypes.c_int
        L.mx_moe_combine.argtypes = [vp, i32, i64, i64, vp, vp, i64, i32, i64, vp, i32, i64, vp]
        L.mx_moe_combine.restype = ctypes.c_int
        L.mx_rmsnorm_quantize.argtypes = [vp, i32, i64, vp, i32, ctypes.c_float, ctypes.POINTER(CMxTensor), i32, vp]
        L.mx_rmsnorm_quantize.restype = ctypes.c_int
        L.mx_workspace_bytes.argtypes = [i32, vp, i32]
        L.mx_workspace_bytes.restype = sz
        L.mx_status_string.argtypes = [ctypes.c_int]
        L.mx_status_string.restype = ctypes.c_char_p
        L.mx_version.argtypes = []
        L.mx_version.restype = ctypes.c_int
        _LIB = L
    return _LIB


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(int(status)).decode()


def mx_version() -> int:
    return lib().mx_version()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MXError(status, where)


def _stream(torch, device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MX_DT_F32
    if t.dtype == torch.bfloat16:
        return MX_DT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class MXTensor:
    """A quantized [rows, cols] tensor: packed codes, scale bytes and (NVFP4)
    the per-tensor fp32 scale, all torch device tensors."""
    fmt: int
    rows: int
    cols: int
    codes: object          # uint8 [rows, cols * bits / 8]
    scales: object         # uint8 [rows, cols/k]
    global_scale: object = None   # float32 [1] (NVFP4)

    def desc(self) -> CMxTensor:
        return CMxTensor(self.fmt, 0, self.rows, self.cols, self.codes.data_ptr(),
                         self.scales.data_ptr() if self.scales is not None else None,
                         self.global_scale.data_ptr() if self.global_scale is not None else None)

    @property
    def block(self) -> int:
        return _BLOCK[self.fmt]


def empty_quantized(rows: int, cols: int, fmt="mxfp4", device="cuda", lead=()) -> MXTensor:
    """Allocate an uninitialised quantized tensor (optionally with leading
    dims, e.g. lead=(G,) for stacked expert weights: rows then means G*N)."""
    import torch
    f = _FMT[fmt] if isinstance(fmt, str) else fmt
    k = _BLOCK[f]
    p = padded_cols(cols, f)
    codes = torch.empty(rows, p * _BITS[f] // 8, dtype=torch.uint8, device=device)
    scales = None if f == MX_FMT_FP4_TENSOR else torch.empty(rows, p // k, dtype=torch.uint8, device=device)
    g = torch.ones(1, dtype=torch.float32, device=device) if f in (MX_FMT_NVFP4, MX_FMT_FP4_TENSOR) else None
    return MXTensor(f, rows, cols, codes, scales, g)


def mx_workspace_bytes(op: int, desc, flags: int = 0) -> int:
    return int(lib().mx_workspace_bytes(op, ctypes.cast(ctypes.pointer(desc), ctypes.c_void_p), flags))


def mx_quantize(x, fmt="mxfp4", out: MXTensor | None = None, static_global=None, workspace=None,
                rule: str = "ceil") -> MXTensor:
    """Quantize a 2-D fp32/bf16 CUDA tensor (row pitch x.stride(0)).
    static_global: NVFP4's calibrated per-tensor scale, or MXFP4_K16's tensor
    scale g.  rule="floor" selects the OCP exponent rule (E8M0 formats)."""
    import torch
    assert x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if out is None:
        out = empty_quantized(rows, cols, fmt, x.device)
    flags = MX_QUANT_DEFAULT
    if static_global is not None:
        if out.global_scale is None:
            out.global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
        out.global_scale.fill_(float(static_global))
        if out.fmt == MX_FMT_NVFP4:
            flags = MX_QUANT_STATIC_GLOBAL
    if rule == "floor":
        flags = MX_QUANT_SCALE_FLOOR
    elif rule != "ceil":
        raise ValueError(rule)
    d = out.desc()
    need = mx_workspace_bytes(MX_OP_QUANTIZE, d, flags)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().mx_quantize(x.data_ptr(), _dt(x), x.stride(0), ctypes.byref(d), flags, ws_ptr, ws_bytes,
                             _stream(torch, x.device)), "mx_quantize")
    return out


def mx_quantize_noalloc(x, out: MXTensor, static_global=None, rule: str = "ceil") -> MXTensor:
    """mx_quantize into a preallocated `out` without a workspace: the library
    keeps the tensor-wide max partials in its static per-device scratch, so
    the call allocates nothing (calls overlapping on one device race)."""
    import torch
    assert x.dim() == 2 and x.stride(1) == 1
    flags = MX_QUANT_DEFAULT
    if static_global is not None:
        out.global_scale.fill_(float(static_global))
        if out.fmt == MX_FMT_NVFP4:
            flags = MX_QUANT_STATIC_GLOBAL
    if rule == "floor":
        flags = MX_QUANT_SCALE_FLOOR
    elif rule != "ceil":
        raise ValueError(rule)
    d = out.desc()
    _check(lib().mx_quantize_noalloc(x.data_ptr(), _dt(x), x.stride(0), ctypes.byref(d), flags,
                                     _stream(torch, x.device)), "mx_quantize_noalloc")
    return out


def mx_dequantize(t: MXTensor, dtype=None, out=None):
    import torch
    dtype = dtype or torch.float32
    if out is None:
        out = torch.empty(t.rows, t.cols, dtype=dtype, device=t.codes.device)
    assert out.dim() == 2 and out.stride(1) == 1, "rows of out must be contiguous"
    d = t.desc()
    _check(lib().mx_dequantize(ctypes.byref(d), out.data_ptr(), _dt(out), out.stride(0),
                               _stream(torch, out.device)), "mx_dequantize")
    return out


def mx_gemm(a, b: MXTensor, N: int | None = None, out_dtype=None, out=None, groups: int = 0, offsets=None,
            a_codes_out=None, a_scales_out=None, workspace=None, f8f6f4_matrix_cores: bool = False,
            fused_quantize: bool = False, a_format=None):
    """C[M, N] = A . B^T.  a is an MXTensor (W4A4) or a raw fp32/bf16 tensor
    (dynamic quantization inside the call, to b's format or to `a_format`,
    e.g. "mxfp8_e4m3").  Grouped: b holds `groups` stacked [N, K] matrices
    and offsets is an int32 CUDA tensor [groups+1].
    f8f6f4_matrix_cores: MX pairs with an FP8/FP6 operand run on the
    block-scaled matrix cores (faster, products truncated) instead of the
    exact route.  fused_quantize: a raw A is quantized inside one persistent
    kernel that also multiplies, instead of in a launch of its own first."""
    import torch
    out_dtype = out_dtype or torch.bfloat16
    if isinstance(a, MXTensor):
        M, K = a.rows, a.cols
        dev = a.codes.device
    else:
        M, K = a.shape
        dev = a.device
    if N is None:
        N = b.rows // max(groups, 1)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=dev)
    bd = b.desc()
    args = CMxGemmArgs()
    args.M, args.N, args.K = M, N, K
    if isinstance(a, MXTensor):
        ad = a.desc()
        args.a = ctypes.pointer(ad)
    else:
        assert a.stride(1) == 1
        args.a = None
        args.a_raw = a.data_ptr()
        args.a_raw_dtype = _dt(a)
        args.lda_raw = a.stride(0)
        if a_codes_out is not None:
            args.a_codes_out = a_codes_out.data_ptr()
            args.a_scales_out = a_scales_out.data_ptr()
    args.groups = groups
    args.b = ctypes.pointer(bd)
    args.group_offsets = offsets.data_ptr() if offsets is not None else None
    assert out.dim() == 2 and out.stride(1) == 1, "rows of out must be contiguous"
    args.c = out.data_ptr()
    args.c_dtype = _dt(out)
    args.flags = ((MX_GEMM_F8F6F4_MATRIX_CORES if f8f6f4_matrix_cores else 0) |
                  (MX_GEMM_FUSED_QUANTIZE if fused_quantize else 0))
    if a_format is not None:
        args.flags |= MX_GEMM_DYNAMIC_A_FORMAT(_FMT[a_format] if isinstance(a_format, str) else a_format)
    args.ldc = out.stride(0)
    need = mx_workspace_bytes(MX_OP_GEMM, args)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    _check(lib().mx_gemm(ctypes.byref(args), _stream(torch, dev)), "mx_gemm")
    return out


def mx_gemv(x, w: MXTensor, out=None):
    """W4A16 (W8A16 / W6A16 for MXFP8 / MXFP6 weights): y[M, N] =
    x[M, K] (bf16) . dequant(w)[N, K]^T, bf16 out, M <= 16."""
    import torch
    M, K = x.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=torch.bfloat16, device=x.device)
    assert x.dim() == 2 and x.stride(1) == 1 and out.stride(1) == 1, "rows of x and out must be contiguous"
    d = w.desc()
    _check(lib().mx_gemv(x.data_ptr(), _dt(x), M, x.stride(0), ctypes.byref(d), out.data_ptr(), _dt(out),
                         out.stride(0), _stream(torch, x.device)), "mx_gemv")
    return out


def mx_moe_route(topk_ids, experts: int, offsets=None, dest_row=None, src_token=None, workspace=None):
    """Stable expert-sorted order of the (token, slot) pairs of an int32 CUDA
    tensor topk_ids [tokens, topk].  Returns (offsets [experts+1],
    dest_row [tokens*topk], src_token [tokens*topk]), int32 CUDA tensors."""
    import torch
    assert topk_ids.dim() == 2 and topk_ids.dtype == torch.int32 and topk_ids.is_contiguous()
    T, k = topk_ids.shape
    dev = topk_ids.device
    if offsets is None:
        offsets = torch.empty(experts + 1, dtype=torch.int32, device=dev)
    if dest_row is None:
        dest_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    if src_token is None:
        src_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    e = ctypes.c_int32(experts)
    need = int(lib().mx_workspace_bytes(MX_OP_MOE_ROUTE, ctypes.cast(ctypes.pointer(e), ctypes.c_void_p), 0))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().mx_moe_route(topk_ids.data_ptr(), T, k, experts, offsets.data_ptr(), dest_row.data_ptr(),
                              src_token.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(torch, dev)),
           "mx_moe_route")
    return offsets, dest_row, src_token


def mx_quantize_rows(x, row_index, out: MXTensor | None = None) -> MXTensor:
    """MXFP4 quantization of the rows x[row_index[r]] (int32 CUDA tensor; an
    index outside [0, x.shape[0]) gives a zero row)."""
    import torch
    assert x.dim() == 2 and x.stride(1) == 1 and row_index.dtype == torch.int32
    R = row_index.numel()
    if out is None:
        out = empty_quantized(R, x.shape[1], "mxfp4", x.device)
    d = out.desc()
    _check(lib().mx_quantize_rows(x.data_ptr(), _dt(x), x.stride(0), x.shape[0], row_index.data_ptr(),
                                  ctypes.byref(d), _stream(torch, x.device)), "mx_quantize_rows")
    return out


def mx_moe_combine(y, dest_row, weights, tokens: int, topk: int, out=None, out_dtype=None):
    """out[t] = sum_s weights[t, s] * y[dest_row[t, s]] (fp32 accumulation)."""
    import torch
    out_dtype = out_dtype or torch.bfloat16
    N = y.shape[1]
    if out is None:
        out = torch.empty(tokens, N, dtype=out_dtype, device=y.device)
    assert y.stride(1) == 1 and out.stride(1) == 1, "rows of y and out must be contiguous"
    _check(lib().mx_moe_combine(y.data_ptr(), _dt(y), y.stride(0), y.shape[0], dest_row.data_ptr(),
                                weights.data_ptr(), tokens, topk, N, out.data_ptr(), _dt(out), out.stride(0),
                                _stream(torch, y.device)), "mx_moe_combine")
    return out


def moe_forward(x, topk_ids, topk_weights, w: MXTensor, experts: int, N: int, y_dtype=None, out_dtype=None,
                bufs: dict | None = None):
    """A routed W4A4 expert layer: mx_moe_route, mx_quantize_rows, grouped
    mx_gemm, mx_moe_combine, in that order on the current stream.  `bufs`
    (optional) holds preallocated intermediates keyed by name."""
    import torch
    y_dtype = y_dtype or torch.bfloat16
    T, k = topk_ids.shape
    b = bufs if bufs is not None else {}
    offsets, dest_row, src_token = mx_moe_route(topk_ids, experts, b.get("offsets"), b.get("dest_row"),
                                                b.get("src_token"), b.get("route_ws"))
    aq = mx_quantize_rows(x, src_token, b.get("aq"))
    y = mx_gemm(aq, w, N=N, out=b.get("y"), out_dtype=y_dtype, groups=experts, offsets=offsets)
    return mx_moe_combine(y, dest_row, topk_weights, T, k, out=b.get("out"), out_dtype=out_dtype)


def mx_rmsnorm_quantize(x, gamma, eps: float = 1e-6, fmt="mxfp4", out: MXTensor | None = None,
                        static_global=None) -> MXTensor:
    """RMSNorm of bf16 rows (gamma fp32/bf16 [K]) quantized in the same kernel
    to MXFP4, or to NVFP4 with the given static per-tensor scale."""
    import torch
    assert x.dim() == 2 and x.stride(1) == 1 and gamma.is_contiguous()
    rows, cols = x.shape
    if out is None:
        out = empty_quantized(rows, cols, fmt, x.device)
    flags = MX_QUANT_DEFAULT
    if static_global is not None:
        out.global_scale.fill_(float(static_global))
        flags = MX_QUANT_STATIC_GLOBAL
    d = out.desc()
    _check(lib().mx_rmsnorm_quantize(x.data_ptr(), _dt(x), x.stride(0), gamma.data_ptr(), _dt(gamma), float(eps),
                                     ctypes.byref(d), flags, _stream(torch, x.device)), "mx_rmsnorm_quantize")
    return out
