"""GPU parity of the fused RMSNorm + FP4 quantization against the CPU oracle.

The oracle is RMSNorm by its definition in fp64; the kernel computes in fp32
(a sum of squares over at most 128 sequential additions per thread and eight
tree levels, r = fp32(1/sqrt(s/K + eps)), then two rounded products), so its
normalized values lie within a relative 72 * 2^-24 of the oracle's (bound
REL below, with margin).  Codes and scale bytes must be identical wherever
that bound cannot move the decision; decisions within the bound of a
boundary (rmsnorm_fragile) are excluded, counted, and required to be rare.
With rows whose squares sum exactly in fp32 (any order gives the same sum)
the bound shrinks to the final roundings (REL_EXACT)."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_mx_amd as mx
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = 2.0 ** -17          # >= (136 / 2 + 3 + 1) * 2^-24
REL_EXACT = 2.0 ** -21    # exact sum of squares: r and two products rounded


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


def check_against_definition(x_bf16, gamma_vals, eps, fmt, g, got_codes, got_scales, rel, what, max_frac=2e-3):
    xv = x_bf16.float().numpy()
    y64 = O.rmsnorm_values(xv, gamma_vals, np.float32(eps))
    rc, rs = O.rmsnorm_quantize(xv, gamma_vals, np.float32(eps), fmt, global_scale=g)
    block, elem = O.rmsnorm_fragile(y64, rel, fmt, g)
    k = 32 if fmt == "mxfp4" else 16
    firm = ~(np.repeat(block, k, axis=1) | elem)
    gc, rcu = O.unpack_codes(got_codes), O.unpack_codes(rc)
    bad_s = (got_scales != rs) & ~block
    bad_c = (gc != rcu) & firm
    assert not bad_s.any(), f"{what}: scale byte differs at a firm block {tuple(np.argwhere(bad_s)[0])}"
    if bad_c.any():
        i = tuple(np.argwhere(bad_c)[0])
        raise AssertionError(f"{what}: code differs at a firm element {i}: gpu={gc[i]} oracle={rcu[i]} y={y64[i]}")
    nfrag = int((~firm).sum())
    ndiff = int(((gc != rcu) | np.repeat(got_scales != rs, k, axis=1)).sum())
    announce(f"{what}: {firm.size - nfrag} firm codes identical; {nfrag} near a boundary ({ndiff} differ)")
    assert nfrag <= max_frac * firm.size, f"{what}: {nfrag} fragile decisions of {firm.size}"


# (1030, 256): more rows than workgroups, so workgroups walk three rows and
# both register sets of the row pipeline are used
@pytest.mark.parametrize("R,K", [(5, 256), (64, 8192), (7, 14336), (3, 32768), (300, 96), (1, 32), (1030, 256)])
@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_rmsnorm_quantize_matches_definition(R, K, gdt, fmt):
    announce(f"rmsnorm quantize R={R} K={K} gamma={gdt} fmt={fmt}")
    rng = np.random.default_rng(R * 13 + K)
    x = (rng.standard_normal((R, K)) * rng.uniform(0.05, 30, (R, 1))).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 60          # outlier channels
    x[0] = 0.0                                  # an all-zero row
    x = torch.from_numpy(x).to(torch.bfloat16)
    gamma = rng.uniform(-1.5, 2.5, K).astype(np.float32)
    gt = torch.from_numpy(gamma).to(gdt)
    eps = 1e-5
    g = np.float32(0.004) if fmt == "nvfp4" else None
    t = mx.mx_rmsnorm_quantize(x.to(DEV), gt.to(DEV), eps, fmt=fmt, static_global=g)
    check_against_definition(x, gt.float().numpy(), eps, fmt, g, host(t.codes), host(t.scales), REL,
                             f"R={R} K={K} {fmt}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("K", [1024, 8192])
def test_rmsnorm_exact_sum_of_squares(fmt, K):
    """Rows of small integers times a power of two: every square and partial
    sum is exact in fp32, so the kernel's sum equals the exact one in any
    order and only the final roundings remain (tight bound)."""
    announce(f"rmsnorm exact sums K={K} {fmt}")
    rng = np.random.default_rng(K + 3)
    R = 16
    x = (rng.integers(-15, 16, (R, K)) * np.exp2(rng.integers(-6, 6, (R, 1)))).astype(np.float32)
    x[3, :] = 0.0
    x[5, ::7] = 0.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy(), x)
    gamma = rng.uniform(0.25, 2.0, K).astype(np.float32)
    g = np.float32(0.003) if fmt == "nvfp4" else None
    t = mx.mx_rmsnorm_quantize(xt.to(DEV), torch.from_numpy(gamma).to(DEV), 1e-6, fmt=fmt, static_global=g)
    check_against_definition(xt, gamma, 1e-6, fmt, g, host(t.codes), host(t.scales), REL_EXACT,
                             f"exact sums K={K} {fmt}")


def test_rmsnorm_nvfp4_scale_code_range():
    """Per-column gains that drive the static-scale NVFP4 block scale through
    E4M3 subnormal codes 1..7, normal codes and saturation at 0x7E."""
    announce("rmsnorm nvfp4 across the E4M3 scale range")
    rng = np.random.default_rng(11)
    R, K = 32, 4096
    x = torch.from_numpy(rng.standard_normal((R, K)).astype(np.float32)).to(torch.bfloat16)
    gains = np.array([30.0, 1.0, 0.05, 2e-3, 1e-4, 4e-5, 2e-5, 1e-5, 6e-6, 3e-6], np.float64)
    gamma = gains[(np.arange(K) // 16) % len(gains)].astype(np.float32)
    g = np.float32(0.002)
    t = mx.mx_rmsnorm_quantize(x.to(DEV), torch.from_numpy(gamma).to(DEV), 1e-6, fmt="nvfp4", static_global=g)
    sc = host(t.scales)
    assert set(range(1, 8)) <= set(np.unique(sc).tolist()), np.unique(sc)
    assert (sc == 0x7E).any() and (sc > 0x40).any()
    check_against_definition(x, gamma, 1e-6, "nvfp4", g, host(t.codes), sc, REL, "nvfp4 scale range")


def test_rmsnorm_quantize_feeds_gemm():
    """The fused output is an ordinary MXFP4 operand: the GEMM of its codes
    equals the oracle GEMM of those codes within the product tolerance."""
    rng = np.random.default_rng(3)
    M, K, N = 96, 1024, 128
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32))
    a = mx.mx_rmsnorm_quantize(x.to(DEV), gamma.to(DEV), 1e-6)
    w = mx.mx_quantize(torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV))
    c = host(mx.mx_gemm(a, w, out_dtype=torch.float32))
    ah = O.dequantize("mxfp4", host(a.codes), host(a.scales))
    bh = O.dequantize("mxfp4", host(w.codes), host(w.scales))
    ref = O.gemm(ah, bh)
    assert np.all(np.abs(c.astype(np.float64) - ref) <= O.gemm_tolerance(ah, bh))
