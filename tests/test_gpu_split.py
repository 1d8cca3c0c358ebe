"""The block-scaled GEMMs' split of a partly filled last round along K (MXFP4
dense and grouped, NVFP4): the last T % 256 tiles run as up to four K parts
each, whose fp32 partial tiles a second launch adds in part order (times
gA * gB for NVFP4).  It runs when the caller's workspace holds the
partials (the binding asks mx_workspace_bytes and provides them); with a
smaller workspace the plain kernel runs.  Both must lie within the GEMM
tolerance of the fp64 oracle, and the split result must repeat bit for bit."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_mx_amd as mx
import oracle as O

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU)")
    mx.lib()
    yield
    torch.cuda.synchronize()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def within(y, yref, tol, what):
    err = np.abs(y.astype(np.float64) - yref.astype(np.float64))
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} outside tolerance, first at {tuple(np.argwhere(bad)[0])}"
    announce(f"{what}: max err / tol = {(err / np.maximum(tol, 1e-300)).max():.3g}")


def operands(M, N, K, seed, fmt="mxfp4"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, size=max(1, K // 500), replace=False)] *= 40
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    a = mx.mx_quantize(torch.from_numpy(x).cuda(), fmt=fmt)
    b = mx.mx_quantize(torch.from_numpy(w).cuda(), fmt=fmt)
    if fmt == "mxfp4":
        ra, rsa = O.mxfp4_quantize(x)
        rb, rsb = O.mxfp4_quantize(w)
        ah, bh = O.dequantize("mxfp4", ra, rsa), O.dequantize("mxfp4", rb, rsb)
    else:
        ra, rsa, ga = O.nvfp4_quantize(x)
        rb, rsb, gb = O.nvfp4_quantize(w)
        ah, bh = O.dequantize("nvfp4", ra, rsa, ga), O.dequantize("nvfp4", rb, rsb, gb)
    assert np.array_equal(host(a.codes), ra) and np.array_equal(host(b.codes), rb)
    return a, b, ah, bh


# (M, N, K): 2 tiles x 4 K parts (paired scale stages); 4 tiles x 3 parts
# (K % 512 != 0: single stages); 272 tiles on 256 CUs: the last 16 tiles (the
# last tile row) in 4 parts
@pytest.mark.parametrize("fmt,mnk,rows", [("mxfp4", (512, 256, 4096), None), ("mxfp4", (300, 258, 768), None),
                                          ("mxfp4", (4352, 4096, 2048), (4032, 4352)),
                                          ("nvfp4", (512, 256, 2048), None), ("nvfp4", (300, 520, 768), None)])
@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
def test_split_last_round(fmt, mnk, rows, odt):
    M, N, K = mnk
    announce(f"split last round {fmt} M={M} N={N} K={K} out={odt}")
    a, b, ah, bh = operands(M, N, K, seed=M + N + K, fmt=fmt)
    y1 = mx.mx_gemm(a, b, out_dtype=odt)
    y2 = mx.mx_gemm(a, b, out_dtype=odt)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")   # too small for the partials: plain kernel
    y0 = mx.mx_gemm(a, b, out_dtype=odt, workspace=small)
    g1, g2, g0 = host(y1.float()), host(y2.float()), host(y0.float())
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32)), "split result differs between calls"
    r0, r1 = rows if rows else (0, M)
    o = "bf16" if odt == torch.bfloat16 else "f32"
    yref = O.gemm(ah[r0:r1], bh, out=o)
    tol = O.gemm_tolerance(ah[r0:r1], bh, yref, out=o)
    within(g1[r0:r1], yref, tol, f"split {fmt} M={M} N={N} K={K} rows {r0}:{r1}")
    within(g0[r0:r1], yref, tol, f"plain {fmt} M={M} N={N} K={K} rows {r0}:{r1}")
    if rows:   # rows outside the split tiles come from the same whole-tile kernel
        assert np.array_equal(g1[:r0].view(np.uint32), g0[:r0].view(np.uint32))
