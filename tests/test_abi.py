"""C-ABI tests that need no GPU: libmx.so loads, exports every function that
include/mx.h declares, and rejects invalid arguments on the host with the
documented status codes before any HIP call (fake, never-dereferenced
pointers are enough for that)."""
import ctypes
import os
import re

import pytest

import microscaling_fp4_quantization_mx_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def header_functions():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(mx_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = mx.lib()
    names = header_functions()
    assert {"mx_quantize", "mx_dequantize", "mx_gemm", "mx_gemv", "mx_workspace_bytes",
            "mx_status_string", "mx_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_dynamic_symbols_are_c_abi():
    out = os.popen(f"nm -D --defined-only {mx.library_path}").read()
    for n in header_functions():
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_status_strings_and_version():
    for s in range(-8, 1):
        assert mx.mx_status_string(s).startswith(mx.STATUS[s])
    assert "unknown" in mx.mx_status_string(-99)
    assert mx.mx_version() >= 10000


def T(fmt=0, rows=64, cols=256, codes=FAKE, scales=FAKE, g=None):
    return mx.CMxTensor(fmt, 0, rows, cols, codes, scales, g)


def quant(x=FAKE, dt=0, ld=256, t=None, flags=0, ws=None, wsb=0):
    t = t or T()
    return mx.lib().mx_quantize(x, dt, ld, ctypes.byref(t), flags, ws, wsb, None)


def test_quantize_validation():
    L = mx.lib()
    assert L.mx_quantize(FAKE, 0, 256, None, 0, None, 0, None) == -1           # NULL descriptor
    assert quant(x=None) == -1                                                  # NULL input
    assert quant(t=T(codes=None)) == -1
    assert quant(t=T(fmt=9)) == -8                                              # unknown format
    assert quant(dt=5) == -4                                                    # unknown dtype
    assert quant(t=T(fmt=1, cols=40, g=FAKE)) == -5                             # cols % 16 != 0
    assert quant(ld=100) == -2                                                  # ld < cols
    assert quant(t=T(rows=-1)) == -2
    assert quant(x=FAKE + 4) == -3                                              # misaligned input
    assert quant(ld=257) == -3                                                  # misaligned rows
    assert quant(t=T(codes=FAKE + 8)) == -3
    assert quant(flags=1) == -5                                                 # static scale: NVFP4 only
    assert quant(t=T(fmt=1, g=None)) == -1                                      # NVFP4 needs global scale
    assert quant(t=T(fmt=1, g=FAKE)) == -7                                      # no workspace
    assert quant(t=T(fmt=1, g=FAKE), ws=FAKE, wsb=16) == -7                     # too small
    assert quant(t=T(rows=0)) == 0                                              # empty: no-op
    assert quant(t=T(cols=0), x=None) == 0


def test_workspace_query():
    L = mx.lib()
    t = T(fmt=1, g=FAKE)
    assert L.mx_workspace_bytes(0, ctypes.cast(ctypes.pointer(t), ctypes.c_void_p), 0) >= 4 * 256
    assert L.mx_workspace_bytes(0, ctypes.cast(ctypes.pointer(t), ctypes.c_void_p), 1) == 0
    t0 = T()
    assert L.mx_workspace_bytes(0, ctypes.cast(ctypes.pointer(t0), ctypes.c_void_p), 0) == 0
    args = mx.CMxGemmArgs()
    args.M, args.N, args.K = 100, 64, 256
    need = L.mx_workspace_bytes(1, ctypes.cast(ctypes.pointer(args), ctypes.c_void_p), 0)
    assert need >= 100 * 256 // 2 + 100 * 256 // 32
    assert L.mx_workspace_bytes(1, None, 0) == 0


def gemm_args(M=64, N=128, K=256, a=True, fmt=0, groups=0, **kw):
    args = mx.CMxGemmArgs()
    args.M, args.N, args.K = M, N, K
    b = T(fmt, N * max(groups, 1), K, g=FAKE if fmt else None)
    args._keep = [b]
    args.b = ctypes.pointer(b)
    if a:
        at = T(fmt, M, K, g=FAKE if fmt else None)
        args._keep.append(at)
        args.a = ctypes.pointer(at)
    args.groups = groups
    args.c = FAKE
    args.c_dtype = 1
    args.ldc = N
    for k, v in kw.items():
        setattr(args, k, v)
    return args


def call_gemm(args):
    return mx.lib().mx_gemm(ctypes.byref(args), None)


def test_gemm_validation():
    L = mx.lib()
    assert L.mx_gemm(None, None) == -1
    a = gemm_args()
    a.b = None
    assert call_gemm(a) == -1
    assert call_gemm(gemm_args(c=None)) == -1
    assert call_gemm(gemm_args(c=FAKE + 2)) == -3
    assert call_gemm(gemm_args(ldc=10)) == -2
    assert call_gemm(gemm_args(c_dtype=9)) == -4
    assert call_gemm(gemm_args(M=-1)) == -2
    assert call_gemm(gemm_args(flags=4)) == -2                                  # unknown flag bit
    bad = gemm_args()
    bad.b.contents.cols = 128                                 # K mismatch
    assert call_gemm(bad) == -2
    mism = gemm_args()
    mism.a.contents.fmt = 1
    mism.a.contents.global_scale = FAKE
    assert call_gemm(mism) == -8                              # A NVFP4, B MXFP4
    assert call_gemm(gemm_args(groups=2)) == -1               # grouped without offsets
    assert call_gemm(gemm_args(groups=2, fmt=1, group_offsets=FAKE)) == -5
    assert call_gemm(gemm_args(K=48, M=0)) == 0              # K % 32 != 0: zero-padded rows accepted
    assert call_gemm(gemm_args(fmt=1, K=48)) == -5            # NVFP4 GEMM needs K % 32 == 0
    # dynamic activation path
    d = gemm_args(a=False, a_raw=FAKE, a_raw_dtype=1, lda_raw=256)
    assert call_gemm(d) == -7                                 # no workspace
    d = gemm_args(a=False, a_raw=FAKE, a_raw_dtype=1, lda_raw=256, a_codes_out=FAKE)
    assert call_gemm(d) == -1                                 # codes_out without scales_out
    d = gemm_args(a=False, a_raw=None, a_raw_dtype=1, lda_raw=256)
    assert call_gemm(d) == -1
    d = gemm_args(a=False, a_raw=FAKE, a_raw_dtype=3, lda_raw=256)
    assert call_gemm(d) == -4
    d = gemm_args(a=False, fmt=1, a_raw=FAKE, a_raw_dtype=1, lda_raw=256)
    assert call_gemm(d) == -5                                 # dynamic NVFP4 not provided
    assert call_gemm(gemm_args(M=0)) == 0                     # empty: no-op
    assert call_gemm(gemm_args(N=0, ldc=0)) == 0


def test_gemv_validation():
    L = mx.lib()
    w = T(0, 512, 256)

    def gv(x=FAKE, xdt=1, M=1, ldx=256, w=w, y=FAKE, ydt=1, ldy=512):
        return L.mx_gemv(x, xdt, M, ldx, ctypes.byref(w) if w is not None else None, y, ydt, ldy, None)

    assert gv(w=None) == -1
    assert gv(x=None) == -1
    assert gv(y=None) == -1
    assert gv(xdt=0) == -4                                    # activations must be bf16
    assert gv(ydt=0) == -4
    assert gv(M=17) == -5
    assert gv(M=-1) == -2
    assert gv(ldx=100) == -2
    assert gv(ldx=260) == -3
    assert gv(ldy=100) == -2
    assert gv(w=T(1, 512, 256, g=FAKE)) == -5                 # NVFP4 weights not provided
    assert gv(M=0) == 0


def test_dequantize_validation():
    L = mx.lib()
    t = T()
    assert L.mx_dequantize(None, FAKE, 0, 256, None) == -1
    assert L.mx_dequantize(ctypes.byref(t), None, 0, 256, None) == -1
    assert L.mx_dequantize(ctypes.byref(t), FAKE, 2, 256, None) == -4
    assert L.mx_dequantize(ctypes.byref(t), FAKE, 0, 255, None) == -2
    assert L.mx_dequantize(ctypes.byref(t), FAKE + 4, 0, 256, None) == -3


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_LIB", None)
    monkeypatch.setattr(mx, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mx.lib()


def test_moe_validation():
    L = mx.lib()
    ws = FAKE
    # mx_moe_route(ids, tokens, topk, experts, offsets, dest_row, src_token, ws, ws_bytes, stream)
    assert L.mx_moe_route(FAKE, 10, 0, 8, FAKE, FAKE, FAKE, ws, 4096, None) == -2        # topk < 1
    assert L.mx_moe_route(FAKE, 10, 2, 0, FAKE, FAKE, FAKE, ws, 4096, None) == -2        # experts < 1
    assert L.mx_moe_route(FAKE, -1, 2, 8, FAKE, FAKE, FAKE, ws, 4096, None) == -2        # tokens < 0
    assert L.mx_moe_route(FAKE, 1 << 30, 4, 8, FAKE, FAKE, FAKE, ws, 4096, None) == -2   # pairs >= 2^31
    assert L.mx_moe_route(None, 10, 2, 8, FAKE, FAKE, FAKE, ws, 4096, None) == -1
    assert L.mx_moe_route(FAKE, 10, 2, 8, None, FAKE, FAKE, ws, 4096, None) == -1
    assert L.mx_moe_route(FAKE + 2, 10, 2, 8, FAKE, FAKE, FAKE, ws, 4096, None) == -3    # misaligned ids
    assert L.mx_moe_route(FAKE, 10, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == -7         # no workspace
    assert L.mx_moe_route(FAKE, 10, 2, 8, FAKE, FAKE, FAKE, ws, 16, None) == -7          # too small
    for experts, chunks in ((300, 65536 // 300), (8, 8192), (1 << 16, 1)):
        e = ctypes.c_int32(experts)
        need = L.mx_workspace_bytes(mx.MX_OP_MOE_ROUTE, ctypes.cast(ctypes.pointer(e), ctypes.c_void_p), 0)
        assert need == (4 * chunks * experts + 255) // 256 * 256                  # per-chunk counts
        exact = 4 * chunks * experts
        assert L.mx_moe_route(FAKE, 10, 2, experts, FAKE, FAKE, FAKE, ws, exact - 4, None) == -7
    # mx_quantize_rows(x, dtype, ld, x_rows, row_index, out, stream)
    t = T(rows=16, cols=256)
    assert L.mx_quantize_rows(FAKE, 0, 256, 10, None, ctypes.byref(t), None) == -1
    assert L.mx_quantize_rows(FAKE, 0, 256, -1, FAKE, ctypes.byref(t), None) == -2
    assert L.mx_quantize_rows(FAKE, 0, 100, 10, FAKE, ctypes.byref(t), None) == -2       # ld < cols
    nv = T(fmt=1, rows=16, cols=256, g=FAKE)
    assert L.mx_quantize_rows(FAKE, 0, 256, 10, FAKE, ctypes.byref(nv), None) == -5      # MXFP4 only
    # mx_moe_combine(y, ydt, ldy, y_rows, dest, w, tokens, topk, N, out, odt, ldo, stream)
    assert L.mx_moe_combine(FAKE, 1, 64, 10, FAKE, FAKE, 5, 2, 60, FAKE, 1, 64, None) == -5   # N % 8
    assert L.mx_moe_combine(FAKE, 1, 64, 10, FAKE, FAKE, 5, 0, 64, FAKE, 1, 64, None) == -2   # topk < 1
    assert L.mx_moe_combine(FAKE, 1, 64, 10, None, FAKE, 5, 2, 64, FAKE, 1, 64, None) == -1
    assert L.mx_moe_combine(FAKE, 7, 64, 10, FAKE, FAKE, 5, 2, 64, FAKE, 1, 64, None) == -4   # dtype
    assert L.mx_moe_combine(FAKE, 1, 60, 10, FAKE, FAKE, 5, 2, 56, FAKE, 1, 64, None) == -3   # row pitch


def test_rmsnorm_quantize_validation():
    L = mx.lib()
    t = T(rows=16, cols=256)
    f = ctypes.c_float
    assert L.mx_rmsnorm_quantize(FAKE, 0, 256, FAKE, 0, f(1e-6), ctypes.byref(t), 0, None) == -4   # x must be bf16
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, FAKE, 9, f(1e-6), ctypes.byref(t), 0, None) == -4   # gamma dtype
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, FAKE, 0, f(0.0), ctypes.byref(t), 0, None) == -2    # eps > 0
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, None, 0, f(1e-6), ctypes.byref(t), 0, None) == -1
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, FAKE, 0, f(1e-6), ctypes.byref(t), 1, None) == -5   # MXFP4: no flags
    nv = T(fmt=1, rows=16, cols=256, g=FAKE)
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, FAKE, 0, f(1e-6), ctypes.byref(nv), 0, None) == -5  # NVFP4: static only
    big = T(rows=2, cols=32768 + 32)
    assert L.mx_rmsnorm_quantize(FAKE, 1, 32800, FAKE, 0, f(1e-6), ctypes.byref(big), 0, None) == -5


def test_variant_format_validation():
    """Emulation variants: MXFP4_K16 (E8M0 per 16, optional tensor scale),
    FP4_TENSOR (one fp32 scale), the floor-rule flag, ragged rows."""
    L = mx.lib()
    assert quant(t=T(fmt=7, g=None)) == -1                                  # FP4_TENSOR needs its scale
    assert quant(t=T(fmt=7, g=FAKE)) == -7                                  # ... and a workspace
    assert quant(t=T(fmt=7, cols=255, g=FAKE), ld=256) == -5                # odd cols
    assert quant(t=T(fmt=7, g=FAKE), flags=2) == -5                         # no floor rule
    assert quant(t=T(fmt=6, g=FAKE), flags=2) == -5                         # floor rule has no tensor scale
    assert quant(t=T(fmt=6), flags=1) == -5                                 # static flag is NVFP4's
    assert quant(t=T(fmt=1, g=FAKE), flags=2) == -5                         # NVFP4: no floor rule
    assert quant(t=T(fmt=1, cols=40, g=FAKE), ld=48) == -5                  # NVFP4 rows stay whole
    assert quant(t=T(fmt=0, rows=0, cols=50), ld=56) == 0                    # ragged MXFP4: accepted (empty)
    assert quant(t=T(fmt=6, rows=0, cols=7), ld=8) == 0
    # GEMM: variants are not matrix-core formats; ragged K with dynamic A is not provided
    g = gemm_args(K=256, fmt=6)
    assert call_gemm(g) == -5
    g = gemm_args(K=256)
    g.a.contents.fmt = 7
    g.a.contents.global_scale = FAKE
    assert call_gemm(g) == -5
    d = gemm_args(a=False, a_raw=FAKE, a_raw_dtype=1, lda_raw=264, K=250, ldc=128)
    assert call_gemm(d) == -5
    # GEMV, gathered quantize: whole blocks only
    w = T(0, 512, 250)
    assert L.mx_gemv(FAKE, 1, 1, 256, ctypes.byref(w), FAKE, 1, 512, None) == -5
    t = T(fmt=0, rows=16, cols=250)
    assert L.mx_quantize_rows(FAKE, 0, 256, 10, FAKE, ctypes.byref(t), None) == -5
    t7 = T(fmt=7, g=FAKE)
    assert L.mx_workspace_bytes(mx.MX_OP_QUANTIZE, ctypes.cast(ctypes.pointer(t7), ctypes.c_void_p), 0) >= 4096


def test_wide_format_validation():
    """MXFP8 / MXFP6 descriptors: quantize and dequantize accept them, the
    GEMM takes any MX pair (dense or grouped, pre-quantized or dynamic A,
    K % 128 == 0), the GEMV takes them as weights, and the remaining entry
    points report them unsupported."""
    L = mx.lib()
    for f in (2, 3, 4, 5):
        assert quant(t=T(fmt=f), flags=1) == -5                            # no static-scale flag
        assert quant(t=T(fmt=f, rows=0)) == 0
        assert L.mx_dequantize(ctypes.byref(T(fmt=f)), FAKE + 4, 0, 256, None) == -3
    # mixed pair A MXFP8 E4M3 x B MXFP4, then the reverse
    g = gemm_args(K=256)
    g.a.contents.fmt = 2
    g.c = None
    assert call_gemm(g) == -1                                              # validation reaches the wide path
    g = gemm_args(K=192)
    g.a.contents.fmt = 2
    assert call_gemm(g) == -5                                              # K % 128
    g = gemm_args(K=256, fmt=4)
    g.a.contents.fmt = 1
    g.a.contents.global_scale = FAKE
    assert call_gemm(g) == -8                                              # NVFP4 x MXFP6
    # grouped wide pairs: the grouped checks apply
    g = gemm_args(K=256, fmt=3, groups=2)
    assert call_gemm(g) == -1                                              # offsets missing
    g = gemm_args(K=256, fmt=3, groups=2, group_offsets=FAKE)
    g.b.contents.rows = 128
    assert call_gemm(g) == -2                                              # b rows != groups * N
    assert call_gemm(gemm_args(M=0, fmt=3, groups=2, group_offsets=FAKE)) == 0
    # dynamic A to a wide format (B's, or the one named in flags)
    dyn = dict(a=False, a_raw=FAKE, a_raw_dtype=1, lda_raw=256)
    assert call_gemm(gemm_args(K=256, fmt=5, **dyn, workspace=None)) == -7  # needs a workspace
    g = gemm_args(K=256, fmt=5, **dyn)
    need = L.mx_workspace_bytes(mx.MX_OP_GEMM, ctypes.cast(ctypes.pointer(g), ctypes.c_void_p), 0)
    assert need == 64 * 256 * 6 // 8 + 64 * 256 // 32                        # E3M2 codes + scale bytes
    g = gemm_args(K=256, fmt=0, **dyn, flags=mx.MX_GEMM_DYNAMIC_A_FORMAT(2))
    need = L.mx_workspace_bytes(mx.MX_OP_GEMM, ctypes.cast(ctypes.pointer(g), ctypes.c_void_p), 0)
    assert need == 64 * 256 + 64 * 256 // 32                                 # E4M3 activations
    assert call_gemm(gemm_args(K=250, fmt=2, **dyn, ldc=128)) == -5         # whole blocks only
    assert call_gemm(gemm_args(K=256, fmt=0, **dyn, flags=mx.MX_GEMM_DYNAMIC_A_FORMAT(1))) == -8   # NVFP4
    assert call_gemm(gemm_args(K=256, fmt=0, **dyn, flags=mx.MX_GEMM_DYNAMIC_A_FORMAT(6))) == -8   # K16 variant
    assert call_gemm(gemm_args(K=256, fmt=0, flags=mx.MX_GEMM_DYNAMIC_A_FORMAT(2))) == -8          # A given
    assert call_gemm(gemm_args(M=0, fmt=2)) == 0
    # GEMV: MXFP8 / MXFP6 weights, whole blocks; not the variants
    w = T(3, 512, 250)
    assert L.mx_gemv(FAKE, 1, 1, 256, ctypes.byref(w), FAKE, 1, 512, None) == -5
    w = T(6, 512, 256)
    assert L.mx_gemv(FAKE, 1, 1, 256, ctypes.byref(w), FAKE, 1, 512, None) == -5
    w = T(4, 512, 256)
    assert L.mx_gemv(FAKE, 1, 17, 256, ctypes.byref(w), FAKE, 1, 512, None) == -5   # M <= 16
    assert L.mx_gemv(FAKE, 1, 0, 256, ctypes.byref(w), FAKE, 1, 512, None) == 0
    t = T(fmt=4, rows=16, cols=256)
    assert L.mx_rmsnorm_quantize(FAKE, 1, 256, FAKE, 0, ctypes.c_float(1e-6), ctypes.byref(t), 0, None) == -5
    assert L.mx_quantize_rows(FAKE, 0, 256, 10, FAKE, ctypes.byref(t), None) == -5


def test_quantize_noalloc_validation():
    """The allocation-free quantize checks every argument before its first HIP
    call (the scratch lookup), with mx_quantize's status codes."""
    L = mx.lib()

    def qn(x=FAKE, dt=0, ld=256, t=None, flags=0):
        t = t or T()
        return L.mx_quantize_noalloc(x, dt, ld, ctypes.byref(t), flags, None)
    assert L.mx_quantize_noalloc(FAKE, 0, 256, None, 0, None) == -1
    assert qn(t=T(fmt=1, g=FAKE), x=None) == -1                             # NVFP4: NULL input
    assert qn(t=T(fmt=1, cols=40, g=FAKE)) == -5                            # cols % 16 != 0
    assert qn(t=T(fmt=1, g=FAKE), x=FAKE + 4) == -3                         # misaligned input
    assert qn(t=T(fmt=1, g=FAKE), dt=7) == -4
    assert qn(t=T(fmt=7, scales=None, g=FAKE), ld=100) == -2                # naive: ld < cols
    assert qn(t=T(fmt=1, g=FAKE, rows=0)) == 0                              # empty: no-op, no HIP call
    assert qn(flags=1) == -5                                                # static scale: NVFP4 only
