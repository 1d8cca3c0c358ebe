"""GPU parity of the fused RMSNorm + FP4 quantization against the CPU oracle:
codes and scale bytes bit for bit (the normalization follows the fixed fp32
order both sides define)."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_mx_amd as mx
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


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


@pytest.mark.parametrize("R,K", [(5, 256), (64, 8192), (7, 14336), (3, 32768), (300, 96), (1, 32)])
@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_rmsnorm_quantize_bit_exact(R, K, gdt, fmt):
    announce(f"rmsnorm quantize R={R} K={K} gamma={gdt} fmt={fmt}")
    rng = np.random.default_rng(R * 13 + K)
    x = (rng.standard_normal((R, K)) * rng.uniform(0.05, 30, (R, 1))).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 60          # outlier channels
    x[0] = 0.0                                  # an all-zero row
    x = torch.from_numpy(x).to(torch.bfloat16)
    gamma = rng.uniform(-1.5, 2.5, K).astype(np.float32)
    gt = torch.from_numpy(gamma).to(gdt)
    gamma_vals = gt.float().numpy()
    eps = 1e-5
    g = np.float32(0.004) if fmt == "nvfp4" else None
    t = mx.mx_rmsnorm_quantize(x.to(DEV), gt.to(DEV), eps, fmt=fmt, static_global=g)
    rc, rs = O.rmsnorm_quantize(x.float().numpy(), gamma_vals, eps, fmt, global_scale=g)
    assert np.array_equal(host(t.codes), rc)
    assert np.array_equal(host(t.scales), rs)


def test_rmsnorm_quantize_feeds_gemm():
    """The fused output is an ordinary MXFP4 operand: its GEMM equals the GEMM
    of mx_quantize applied to the oracle's normalized values."""
    rng = np.random.default_rng(3)
    M, K, N = 96, 1024, 128
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32))
    a = mx.mx_rmsnorm_quantize(x.to(DEV), gamma.to(DEV), 1e-6)
    y = O.rmsnorm_values(x.float().numpy(), gamma.numpy(), 1e-6)
    a2 = mx.mx_quantize(torch.from_numpy(y).to(DEV))
    w = mx.mx_quantize(torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV))
    c1 = mx.mx_gemm(a, w, out_dtype=torch.float32)
    c2 = mx.mx_gemm(a2, w, out_dtype=torch.float32)
    assert torch.equal(c1, c2)
