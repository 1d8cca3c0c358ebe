"""GPU parity of the wider MX elements (MXFP8 E4M3/E5M2, MXFP6 E2M3/E3M2)
against the CPU oracle: codes and scale bytes bit for bit, dequantized values
exactly, and block-scaled products of every MX format pair (mixed pairs
included) within the bound of the matrix-core arithmetic.

The bound: 1e-5 * sum_k |a_k b_k| for the fp32 accumulation (+ one bf16 ulp
for bf16 output), plus the truncation inside the block-scaled MFMA.  Measured
with exact test values on the hardware: the products of each group of 8
consecutive K are summed after each product is truncated toward zero at 13
bits below the leading bit of the group's largest product (FP6 pairs keep at
least that many).  So a product loses less than 2^(L - 13), L = floor(log2 of
the group's largest |product|), and a group of 8 less than 8 * 2^(L + 1 - 13)
(one bit of slack for the product's leading bit).  E2M1 x E2M1 products span
7 bits and lose nothing."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_mx_amd as mx
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
WIDE = ["mxfp8_e4m3", "mxfp8_e5m2", "mxfp6_e2m3", "mxfp6_e3m2"]
ALL = WIDE + ["mxfp4"]


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


def bf16_values(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def hard_inputs(rows, cols, seed, fmt):
    """Gaussian rows over a wide exponent range plus the cases that decide
    codes: an all-zero block, signed zeros, a large outlier, tiny values,
    and a block of exact half-way points between neighbouring states."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-24, 24, (rows, 1)))).astype(np.float32)
    if rows >= 4 and cols >= 64:
        x[0, :32] = 0.0
        x[1, 3:9] = -0.0
        x[2, 40] = x[2, 40] * 3e4
        x[3, 32:64] = rng.standard_normal(32).astype(np.float32) * 1e-30
    if rows >= 5 and cols >= 32:
        t = O.element_positive_values(fmt)
        mids = (t[:-1] + t[1:]) / 2
        k = min(31, len(mids))
        sel = mids[np.linspace(0, len(mids) - 1, k).astype(int)]
        blk = np.concatenate([[t[-1]], sel])[:32] * 2.0 ** 5
        blk = np.pad(blk, (0, 32 - len(blk)))
        x[4, :32] = (blk * np.where(np.arange(32) % 3 == 0, -1, 1)).astype(np.float32)
    return x


@pytest.mark.parametrize("fmt", WIDE)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols,pad", [(1, 32, 0), (37, 96, 0), (130, 1024, 0), (9, 160, 32)])
def test_wide_quantize_bit_exact(fmt, dtype, rows, cols, pad):
    announce(f"wide quantize {fmt} {dtype} {rows}x{cols} pad={pad}")
    x = hard_inputs(rows, cols, rows * 31 + cols, fmt)
    if dtype == torch.bfloat16:
        x = bf16_values(x)
    xt = torch.zeros(rows, cols + pad, dtype=dtype, device=DEV)
    xt[:, :cols] = torch.from_numpy(x).to(dtype).to(DEV)
    q = mx.mx_quantize(xt[:, :cols], fmt)
    rc, rs = O.mx_quantize_fmt(x, fmt)
    gc, gs = host(q.codes), host(q.scales)
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:5]
    assert np.array_equal(gc, rc), np.argwhere(gc != rc)[:5]


@pytest.mark.parametrize("fmt", WIDE)
def test_wide_dequantize_exact(fmt):
    announce(f"wide dequantize {fmt}")
    x = hard_inputs(21, 320, 7, fmt)
    q = mx.mx_quantize(torch.from_numpy(x).to(DEV), fmt)
    ref = O.dequantize_fmt(fmt, host(q.codes), host(q.scales))
    assert np.array_equal(host(mx.mx_dequantize(q)), ref)
    yb = mx.mx_dequantize(q, torch.bfloat16)
    assert np.array_equal(host(yb.float()), bf16_values(ref))
    # strided output rows
    out = torch.full((21, 352), 7.0, device=DEV)
    mx.mx_dequantize(q, out=out[:, :320])
    got = host(out)
    assert np.array_equal(got[:, :320], ref) and np.all(got[:, 320:] == 7.0)


MFMA_KEEP_BITS = 13
MFMA_GROUP = 8


def mfma_truncation_bound(ah, bh, keep=MFMA_KEEP_BITS, group=MFMA_GROUP, rows_per_chunk=8):
    """sum over groups g of `group` consecutive k of group * 2^(L_g + 1 - keep),
    L_g = floor(log2 max_{k in g} |a_k b_k|) (0 for an all-zero group)."""
    ah = np.asarray(ah, np.float64)
    bh = np.asarray(bh, np.float64)
    M, K = ah.shape
    out = np.zeros((M, bh.shape[0]))
    for r0 in range(0, M, rows_per_chunk):
        p = np.abs(ah[r0:r0 + rows_per_chunk, None, :] * bh[None, :, :])
        gm = p.reshape(p.shape[0], p.shape[1], K // group, group).max(-1)
        with np.errstate(divide="ignore"):
            lead = np.floor(np.log2(gm))
        out[r0:r0 + rows_per_chunk] = np.where(gm > 0, group * np.exp2(lead + 1 - keep), 0.0).sum(-1)
    return out


def _gemm_case(fa, fb, M, N, K, out_dtype, seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, 1)))).astype(np.float32)
    a[:, 5] *= 40.0                                           # an outlier channel
    b = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    qa = mx.mx_quantize(torch.from_numpy(a).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), fb)
    c = mx.mx_gemm(qa, qb, out_dtype=out_dtype)
    ah = O.dequantize_fmt(fa, host(qa.codes), host(qa.scales))
    bh = O.dequantize_fmt(fb, host(qb.codes), host(qb.scales))
    out = "bf16" if out_dtype == torch.bfloat16 else "f32"
    ref = O.gemm(ah, bh, out=out)
    tol = O.gemm_tolerance(ah, bh, ref, out=out) + mfma_truncation_bound(ah, bh)
    got = host(c.float()).astype(np.float64)
    return got, ref.astype(np.float64), tol


PAIRS = [(fa, fb) for fa in ALL for fb in ALL if (fa, fb) != ("mxfp4", "mxfp4")]


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_wide_gemm_pairs(fa, fb):
    out_dtype = torch.bfloat16 if (ALL.index(fa) + ALL.index(fb)) % 2 else torch.float32
    announce(f"wide gemm {fa} x {fb} 300x260x384 out={out_dtype}")
    got, ref, tol = _gemm_case(fa, fb, 300, 260, 384, out_dtype, seed=ALL.index(fa) * 5 + ALL.index(fb))
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(got - ref).max())


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 257, 256), (513, 7, 128), (256, 256, 1024)])
def test_wide_gemm_edges(M, N, K):
    announce(f"wide gemm edges mxfp8_e4m3 x mxfp4 {M}x{N}x{K}")
    got, ref, tol = _gemm_case("mxfp8_e4m3", "mxfp4", M, N, K, torch.float32, seed=M + N + K)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


def test_wide_gemm_multi_tile():
    announce("wide gemm mxfp8_e5m2 x mxfp6_e3m2 1024x768x2048")
    got, ref, tol = _gemm_case("mxfp8_e5m2", "mxfp6_e3m2", 1024, 768, 2048, torch.bfloat16, seed=3)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


@pytest.mark.parametrize("fa,fb", list(W.WIDE_PAIRS))
def test_wide_gemm_full_size_sampled(fa, fb):
    """The benchmark's 4096 x 8192 x 8192 products in their launch
    configuration; sampled rows and columns against the oracle."""
    w = W.WIDE
    announce(f"wide gemm full size {fa} x {fb} {w.M}x{w.N}x{w.K}")
    d = W.make(w)
    qa = mx.mx_quantize(torch.from_numpy(d["x"]).to(torch.bfloat16).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(d["w"]).to(DEV), fb)
    c = mx.mx_gemm(qa, qb, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(17)
    rows = np.sort(rng.choice(w.M, 12, replace=False))
    cols = np.sort(rng.choice(w.N, 40, replace=False))
    ca, sa = O.mx_quantize_fmt(d["x"][rows], fa)
    assert np.array_equal(host(qa.codes)[rows], ca) and np.array_equal(host(qa.scales)[rows], sa)
    ah = O.dequantize_fmt(fa, ca, sa)
    bh = O.dequantize_fmt(fb, host(qb.codes)[cols], host(qb.scales)[cols])
    ref = O.gemm(ah, bh, out="bf16").astype(np.float64)
    tol = O.gemm_tolerance(ah, bh, ref, out="bf16") + mfma_truncation_bound(ah, bh)
    got = host(c.float())[np.ix_(rows, cols)].astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_wide_gemm_exact_structured(fa, fb):
    """Integers 1..3 (signed) times a power of two per 32-element block, in
    every format exactly: products span 4 bits, so nothing is truncated, and
    every partial sum is exact in fp32 -- the result must equal the exact
    product bit for bit.  Any misplaced element or block scale shows."""
    announce(f"wide gemm exact {fa} x {fb} 130x200x384")
    rng = np.random.default_rng(ALL.index(fa) * 7 + ALL.index(fb))
    M, N, K = 130, 200, 384

    def make(rows, lo, hi):
        v = rng.integers(-3, 4, (rows, K)).astype(np.float64)
        v *= np.repeat(np.exp2(rng.integers(lo, hi + 1, (rows, K // 32))), 32, axis=1)
        return v.astype(np.float32)

    a, b = make(M, -3, 3), make(N, -2, 2)
    qa = mx.mx_quantize(torch.from_numpy(a).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), fb)
    assert np.array_equal(O.dequantize_fmt(fa, host(qa.codes), host(qa.scales)), a)
    assert np.array_equal(O.dequantize_fmt(fb, host(qb.codes), host(qb.scales)), b)
    c = host(mx.mx_gemm(qa, qb, out_dtype=torch.float32)).astype(np.float64)
    assert np.array_equal(c, a.astype(np.float64) @ b.astype(np.float64).T)
