"""GPU parity of the wider MX elements (MXFP8 E4M3/E5M2, MXFP6 E2M3/E3M2)
against the CPU oracle: codes and scale bytes bit for bit, dequantized values
exactly, and block-scaled products of every MX format pair (mixed pairs
included).

Default (exact) route: within 1e-5 * sum_k |a_k b_k| (+ one bf16 ulp for bf16
output), the same bar as the FP4 GEMM.  Route MX_GEMM_F8F6F4_MATRIX_CORES
(block-scaled matrix cores): that bound plus the truncation those matrix
cores apply -- the products of each group of 8 consecutive K are summed after
each product is truncated toward zero at 13 bits below the leading bit of
the group's largest product, so a product loses less than 2^(L - 13), L =
floor(log2 of the group's largest |product|), and a group of 8 less than
8 * 2^(L + 1 - 13) (one bit of slack for the product's leading bit).
test_f8f6f4_truncation_probe pins that model with exact values.  E2M1 x E2M1
products span 7 bits and lose nothing on either route."""
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
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wide_quantize_every_bf16(fmt, dtype):
    """Every finite bf16 magnitude, both signs, coded at its own block scale
    and at 1, 2, 4, 8 and 12 scale steps above it (subnormal codes, ties and
    underflow to zero): blocks of one scale-setting maximum Emax * 2^e and
    31 values; codes and scale bytes bit-exact against the oracle."""
    announce(f"wide quantize every bf16 {fmt} {dtype}")
    bits = np.arange(1, 0x7F80, dtype=np.uint32)          # positive finite bf16 patterns
    vals = (bits << 16).view(np.float32).astype(np.float64)
    pad = (-len(vals)) % 31
    groups = np.concatenate([vals, vals[:pad]]).reshape(-1, 31)
    groups = groups * np.where(np.arange(31) % 2 == 0, 1.0, -1.0)
    emax = float(O.element_positive_values(fmt)[-1])
    a = np.abs(groups).max(axis=1)
    e0 = np.ceil(np.log2(a / emax))
    e0 = np.where(emax * np.exp2(e0 - 1) >= a, e0 - 1, e0)   # the smallest e with a <= emax 2^e
    rows = []
    for d in (0, 1, 2, 4, 8, 12):
        m = emax * np.exp2(e0 + d)
        ok = m <= 3.3e38                                   # a finite bf16 maximum
        rows.append(np.concatenate([m[ok, None], groups[ok]], axis=1))
    x = np.concatenate(rows).astype(np.float32)
    assert np.array_equal(bf16_values(x), x)
    q = mx.mx_quantize(torch.from_numpy(x).to(dtype).to(DEV), fmt)
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


def _gemm_case(fa, fb, M, N, K, out_dtype, seed, fast=False):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 6, (M, 1)))).astype(np.float32)
    a[:, 5] *= 40.0                                           # an outlier channel
    b = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    qa = mx.mx_quantize(torch.from_numpy(a).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), fb)
    c = mx.mx_gemm(qa, qb, out_dtype=out_dtype, f8f6f4_matrix_cores=fast)
    ah = O.dequantize_fmt(fa, host(qa.codes), host(qa.scales))
    bh = O.dequantize_fmt(fb, host(qb.codes), host(qb.scales))
    out = "bf16" if out_dtype == torch.bfloat16 else "f32"
    ref = O.gemm(ah, bh, out=out)
    tol = O.gemm_tolerance(ah, bh, ref, out=out)
    if fast:
        tol = tol + mfma_truncation_bound(ah, bh)
    got = host(c.float()).astype(np.float64)
    return got, ref.astype(np.float64), tol


PAIRS = [(fa, fb) for fa in ALL for fb in ALL if (fa, fb) != ("mxfp4", "mxfp4")]


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_wide_gemm_pairs(fa, fb, fast):
    out_dtype = torch.bfloat16 if (ALL.index(fa) + ALL.index(fb)) % 2 else torch.float32
    announce(f"wide gemm {fa} x {fb} 300x260x384 out={out_dtype} f8f6f4={fast}")
    got, ref, tol = _gemm_case(fa, fb, 300, 260, 384, out_dtype, seed=ALL.index(fa) * 5 + ALL.index(fb), fast=fast)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(got - ref).max())


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 257, 256), (513, 7, 128), (256, 256, 1024)])
def test_wide_gemm_edges(M, N, K, fast):
    announce(f"wide gemm edges mxfp8_e4m3 x mxfp4 {M}x{N}x{K} f8f6f4={fast}")
    got, ref, tol = _gemm_case("mxfp8_e4m3", "mxfp4", M, N, K, torch.float32, seed=M + N + K, fast=fast)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


@pytest.mark.parametrize("fast", [False, True])
def test_wide_gemm_multi_tile(fast):
    announce(f"wide gemm mxfp8_e5m2 x mxfp6_e3m2 1024x768x2048 f8f6f4={fast}")
    got, ref, tol = _gemm_case("mxfp8_e5m2", "mxfp6_e3m2", 1024, 768, 2048, torch.bfloat16, seed=3, fast=fast)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


def test_f8f6f4_truncation_probe():
    """Exact values that show the block-scaled matrix cores' truncation:
    a = (448, 15/256, 0, ...) in E4M3, b = (1, 1, 0, ...): the exact product
    448 + 15/256 comes out on the exact route; on the f8f6f4 route the second
    product shares a group of 8 K with 448 (leading bit 2^8) and is cut to a
    multiple of 2^(8-13): 448 + 1/32.  Moved to K = 8 (another group), the
    small product is kept exactly by both routes."""
    announce("f8f6f4 truncation probe")
    K = 128
    res = {}
    for k_small in (1, 8):
        a = np.zeros((1, K), np.float32)
        a[0, 0], a[0, k_small] = 448.0, 15.0 / 256.0
        b = np.zeros((1, K), np.float32)
        b[0, 0], b[0, k_small] = 1.0, 1.0
        qa = mx.mx_quantize(torch.from_numpy(a).to(DEV), "mxfp8_e4m3")
        qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), "mxfp8_e4m3")
        assert np.array_equal(O.dequantize_fmt("mxfp8_e4m3", host(qa.codes), host(qa.scales)), a)
        assert np.array_equal(O.dequantize_fmt("mxfp8_e4m3", host(qb.codes), host(qb.scales)), b)
        for fast in (False, True):
            c = mx.mx_gemm(qa, qb, out_dtype=torch.float32, f8f6f4_matrix_cores=fast)
            res[(k_small, fast)] = float(host(c)[0, 0])
    assert res[(1, False)] == 448.0 + 15.0 / 256.0
    assert res[(1, True)] == 448.0 + 1.0 / 32.0
    assert res[(8, False)] == res[(8, True)] == 448.0 + 15.0 / 256.0


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("fa,fb", list(W.WIDE_PAIRS))
def test_wide_gemm_full_size_sampled(fa, fb, fast):
    """The benchmark's 4096 x 8192 x 8192 products in their launch
    configuration; sampled rows and columns against the oracle."""
    w = W.WIDE
    announce(f"wide gemm full size {fa} x {fb} {w.M}x{w.N}x{w.K} f8f6f4={fast}")
    d = W.make(w)
    qa = mx.mx_quantize(torch.from_numpy(d["x"]).to(torch.bfloat16).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(d["w"]).to(DEV), fb)
    c = mx.mx_gemm(qa, qb, out_dtype=torch.bfloat16, f8f6f4_matrix_cores=fast)
    rng = np.random.default_rng(17)
    rows = np.sort(rng.choice(w.M, 12, replace=False))
    cols = np.sort(rng.choice(w.N, 40, replace=False))
    ca, sa = O.mx_quantize_fmt(d["x"][rows], fa)
    assert np.array_equal(host(qa.codes)[rows], ca) and np.array_equal(host(qa.scales)[rows], sa)
    ah = O.dequantize_fmt(fa, ca, sa)
    bh = O.dequantize_fmt(fb, host(qb.codes)[cols], host(qb.scales)[cols])
    ref = O.gemm(ah, bh, out="bf16").astype(np.float64)
    tol = O.gemm_tolerance(ah, bh, ref, out="bf16") + (mfma_truncation_bound(ah, bh) if fast else 0.0)
    got = host(c.float())[np.ix_(rows, cols)].astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_wide_gemm_exact_structured(fa, fb, fast):
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
    c = host(mx.mx_gemm(qa, qb, out_dtype=torch.float32, f8f6f4_matrix_cores=fast)).astype(np.float64)
    assert np.array_equal(c, a.astype(np.float64) @ b.astype(np.float64).T)


# ---------------------------------------------------------------- grouped form
def _grouped_ref(ah, bh_stack, offsets, N, out):
    """Rows [off[g], off[g+1]) of A against matrix g of the stack (oracle gemm
    per group), with the per-element tolerance of each group's product."""
    M = ah.shape[0]
    ref = np.zeros((M, N), np.float64)
    tol = np.zeros((M, N), np.float64)
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        bg = bh_stack[g * N:(g + 1) * N]
        y = O.gemm(ah[r0:r1], bg, out=out)
        ref[r0:r1] = y
        tol[r0:r1] = O.gemm_tolerance(ah[r0:r1], bg, y, out=out)
    return ref, tol


GROUPED_PAIRS = [("mxfp8_e4m3", "mxfp4"), ("mxfp6_e2m3", "mxfp6_e2m3"), ("mxfp4", "mxfp8_e5m2"),
                 ("mxfp8_e5m2", "mxfp6_e3m2")]


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("fa,fb", GROUPED_PAIRS)
def test_wide_grouped_gemm(fa, fb, fast):
    """Four groups with ragged row counts (one empty, one spanning two tile
    rows plus a tail): every row against its own group's matrix."""
    G, N, K = 4, 200, 384
    counts = [300, 0, 41, 260]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    announce(f"wide grouped gemm {fa} x {fb} G={G} M={M} N={N} K={K} f8f6f4={fast}")
    rng = np.random.default_rng(ALL.index(fa) * 7 + ALL.index(fb))
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-4, 4, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((G * N, K)) * 0.05).astype(np.float32)
    qa = mx.mx_quantize(torch.from_numpy(a).to(DEV), fa)
    qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), fb)
    off = torch.from_numpy(offsets).to(DEV)
    c = mx.mx_gemm(qa, qb, N=N, out_dtype=torch.float32, groups=G, offsets=off, f8f6f4_matrix_cores=fast)
    ah = O.dequantize_fmt(fa, host(qa.codes), host(qa.scales))
    bh = O.dequantize_fmt(fb, host(qb.codes), host(qb.scales))
    ref, tol = _grouped_ref(ah, bh, offsets, N, "f32")
    if fast:
        for g in range(G):
            r0, r1 = offsets[g], offsets[g + 1]
            if r1 > r0:
                tol[r0:r1] += mfma_truncation_bound(ah[r0:r1], bh[g * N:(g + 1) * N])
    got = host(c).astype(np.float64)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(got - ref).max())


# ------------------------------------------------ dynamic activation quantize
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("afmt,bfmt", [(None, "mxfp8_e4m3"), (None, "mxfp6_e3m2"), ("mxfp8_e4m3", "mxfp4"),
                                       ("mxfp6_e2m3", "mxfp8_e5m2"), ("mxfp4", "mxfp6_e2m3")])
def test_wide_dynamic_gemm(afmt, bfmt, dtype):
    """Raw activations quantized inside the call, to B's format or to the
    named one: the side-output codes and scale bytes equal the oracle's
    quantization bit for bit, and C is the oracle product of those operands
    (dense, then grouped with the same rows)."""
    fa = afmt or bfmt
    M, N, K = 130, 96, 512
    announce(f"wide dynamic gemm A {fa} (raw {dtype}) x B {bfmt} {M}x{N}x{K}")
    rng = np.random.default_rng(ALL.index(fa) * 11 + ALL.index(bfmt))
    a = hard_inputs(M, K, 5, fa) if dtype == torch.float32 else bf16_values(hard_inputs(M, K, 5, fa))
    a = np.clip(a, -2.0 ** 100, 2.0 ** 100).astype(np.float32)
    b = (rng.standard_normal((2 * N, K)) * 0.05).astype(np.float32)
    qb = mx.mx_quantize(torch.from_numpy(b).to(DEV), bfmt)
    at = torch.from_numpy(a).to(dtype).to(DEV)
    bits = mx.element_bits(mx._FMT[fa])
    codes = torch.empty(M, K * bits // 8, dtype=torch.uint8, device=DEV)
    scales = torch.empty(M, K // 32, dtype=torch.uint8, device=DEV)
    rc, rs = O.mx_quantize_fmt(a, fa)
    ah = O.dequantize_fmt(fa, rc, rs)
    bh = O.dequantize_fmt(bfmt, host(qb.codes), host(qb.scales))
    # dense, against the first N rows of B
    qb_dense = mx.MXTensor(qb.fmt, N, K, qb.codes[:N], qb.scales[:N])
    c = mx.mx_gemm(at, qb_dense, out_dtype=torch.float32, a_codes_out=codes, a_scales_out=scales, a_format=afmt)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)
    ref = O.gemm(ah, bh[:N])
    assert np.all(np.abs(host(c) - ref) <= O.gemm_tolerance(ah, bh[:N]))
    # grouped, A in the workspace
    offsets = np.array([0, 57, M], np.int32)
    c2 = mx.mx_gemm(at, qb, N=N, out_dtype=torch.bfloat16, groups=2, offsets=torch.from_numpy(offsets).to(DEV),
                    a_format=afmt)
    ref2, tol2 = _grouped_ref(ah, bh, offsets, N, "bf16")
    got2 = host(c2.float()).astype(np.float64)
    assert np.all(np.abs(got2 - ref2) <= tol2), np.abs(got2 - ref2).max()


# ----------------------------------------------------------- W8A16 / W6A16 GEMV
@pytest.mark.parametrize("fmt", WIDE)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16])
def test_wide_gemv(fmt, M):
    """MXFP8 / MXFP6 weights with bf16 activations: N = 300 (a ragged last
    workgroup of 32 rows), K = 4160 (two full 2048-element windows and a
    partial third)."""
    N, K = 300, 4160
    announce(f"wide gemv {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 13 + WIDE.index(fmt))
    x = bf16_values(rng.standard_normal((M, K)).astype(np.float32) * 2)
    w = hard_inputs(N, K, M + 1, fmt) * np.float32(1e-3)
    wq = mx.mx_quantize(torch.from_numpy(w).to(DEV), fmt)
    wh = O.dequantize_fmt(fmt, host(wq.codes), host(wq.scales))
    y = host(mx.mx_gemv(torch.from_numpy(x).to(torch.bfloat16).to(DEV), wq).float()).astype(np.float64)
    yref = O.gemm(x, wh, out="bf16")
    tol = O.gemm_tolerance(x, wh, yref, out="bf16")
    bad = np.abs(y - yref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(y - yref).max())


@pytest.mark.parametrize("fmt", WIDE)
@pytest.mark.parametrize("M,N,K", [(4, 300, 4096), (5, 70, 768), (8, 33, 256), (11, 96, 2560), (16, 300, 1280)])
def test_wide_gemv_matrix_cores(fmt, M, N, K):
    """4 <= M <= 16 with K a multiple of 256 (the matrix-core kernel): ragged
    last workgroups of 32 rows, chunks of 512 elements with a half chunk at
    the end (768, 2560, 1280), a single chunk (256), 8 and 16 staged rows."""
    announce(f"wide gemv matrix cores {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 17 + N + K + WIDE.index(fmt))
    x = bf16_values(rng.standard_normal((M, K)).astype(np.float32) * 2)
    w = hard_inputs(N, K, M + 3, fmt) * np.float32(1e-3)
    wq = mx.mx_quantize(torch.from_numpy(w).to(DEV), fmt)
    wh = O.dequantize_fmt(fmt, host(wq.codes), host(wq.scales))
    y = host(mx.mx_gemv(torch.from_numpy(x).to(torch.bfloat16).to(DEV), wq).float()).astype(np.float64)
    yref = O.gemm(x, wh, out="bf16")
    tol = O.gemm_tolerance(x, wh, yref, out="bf16")
    bad = np.abs(y - yref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(y - yref).max())


@pytest.mark.parametrize("fmt", ["mxfp8_e4m3", "mxfp6_e3m2"])
def test_wide_gemv_strided(fmt):
    """Activation and output rows as column slices of wider tensors."""
    M, N, K = 8, 64, 1024
    announce(f"wide gemv strided {fmt}")
    rng = np.random.default_rng(99)
    x = bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    wq = mx.mx_quantize(torch.from_numpy(w).to(DEV), fmt)
    wh = O.dequantize_fmt(fmt, host(wq.codes), host(wq.scales))
    xw = torch.zeros(M, K + 128, dtype=torch.bfloat16, device=DEV)
    xw[:, :K] = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    xw[:, K:] = float("nan")                      # never read
    yw = torch.full((M, N + 32), -1.0, dtype=torch.bfloat16, device=DEV)
    mx.mx_gemv(xw[:, :K], wq, out=yw[:, :N])
    got = host(yw.float()).astype(np.float64)
    yref = O.gemm(x, wh, out="bf16")
    assert np.all(np.abs(got[:, :N] - yref) <= O.gemm_tolerance(x, wh, yref, out="bf16"))
    assert np.all(got[:, N:] == -1.0)


@pytest.mark.parametrize("fmt", ["mxfp8_e5m2", "mxfp6_e3m2"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (4, 33, 64), (16, 7, 2080)])
def test_wide_gemv_edges(fmt, M, N, K):
    """One-block rows, a single output column, N below one workgroup's rows,
    K one block past a 2048-element window."""
    announce(f"wide gemv edges {fmt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N + K)
    x = bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    w = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    wq = mx.mx_quantize(torch.from_numpy(w).to(DEV), fmt)
    wh = O.dequantize_fmt(fmt, host(wq.codes), host(wq.scales))
    y = host(mx.mx_gemv(torch.from_numpy(x).to(torch.bfloat16).to(DEV), wq).float()).astype(np.float64)
    yref = O.gemm(x, wh, out="bf16")
    assert np.all(np.abs(y - yref) <= O.gemm_tolerance(x, wh, yref, out="bf16")), np.abs(y - yref).max()
