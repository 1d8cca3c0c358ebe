"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/, each file cites its page and table/figure),
brute force in exact rational arithmetic, closed forms, invariants and
library routines (torch's float8_e4m3fn / bfloat16 casts, numpy int64 matmul).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- exact helpers
E2M1_FR = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
           Fraction(3), Fraction(4), Fraction(6)]


def bf_nearest_e2m1(v: Fraction) -> int:
    """Brute force: index of the nearest of the 8 states to v >= 0 (exact),
    half-way cases to the even index; everything above 6 takes 6."""
    best, bd = None, None
    for i, t in enumerate(E2M1_FR):
        d = abs(v - t)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


def e4m3_fr(code: int) -> Fraction:
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 64)
    return Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


E4M3_FR = [e4m3_fr(c) for c in range(0x7F)]


def bf_nearest_e4m3(r: Fraction) -> int:
    best, bd = None, None
    for c, val in enumerate(E4M3_FR):
        d = abs(r - val)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best


def bf_block_exponent(m: Fraction) -> int:
    """Smallest integer e with m <= 6 * 2^e, after the emulation's guard
    m >= 1e-8 (fp32)."""
    m = max(m, Fraction(float(np.float32(1e-8))))
    e = -200
    while 6 * Fraction(2) ** e < m:
        e += 1
    return e


def bf_mxfp4_block(xs, block_exp_override=None):
    """Brute-force MXFP4 of one block (list of fp32 floats) -> (codes, E8M0 byte)."""
    m = max(abs(Fraction(float(x))) for x in xs)
    e = bf_block_exponent(m)
    codes = []
    for x in xs:
        v = abs(Fraction(float(x))) / Fraction(2) ** e
        c = bf_nearest_e2m1(v)
        if np.signbit(np.float32(x)):
            c |= 8
        codes.append(c)
    return codes, e + 127


# ------------------------------------------------------------------- P1: E2M1
def test_e2m1_table_matches_page():
    rows = _rows("e2m1_table.txt")
    assert len(rows) == 8
    for bits, sign, exp, man, val in rows:
        code = int(bits, 2)
        assert sign == "+" and bits[1:3] == exp and bits[3] == man
        assert O.E2M1_POSITIVE[code] == float(val)
        assert O.e2m1_value_from_bits(code) == float(val)          # bit-field formula
        assert O.e2m1_value_from_bits(code | 8) == -float(val)     # mirror
    assert np.signbit(O.e2m1_value_from_bits(8)) and O.e2m1_value_from_bits(8) == 0.0  # -0


def test_e2m1_decode_vector_equals_bitfields():
    codes = np.arange(16)
    dec = O.e2m1_decode(codes)
    ref = np.array([O.e2m1_value_from_bits(int(c)) for c in codes])
    assert np.array_equal(dec, ref) and np.array_equal(np.signbit(dec), np.signbit(ref))


# ------------------------------------------------------------------- P2: storage
def test_storage_closed_form_matches_pages():
    rows = _rows("storage_footprint.txt")
    d = {(r[0], r[1]): float(r[2]) for r in rows}
    # 16 elements: 16 * 4 + 8 bits
    assert 16 * 4 + 8 == d[("bits_per_block16", "72")]
    R, K = 64, 4096
    nv = O.storage_bytes(R, K, "nvfp4") - 4          # minus the per-tensor fp32
    mx = O.storage_bytes(R, K, "mxfp4")
    assert nv * 8 / (R * K) == d[("bits_per_elem", "block16_8bit_scale")]
    assert mx * 8 / (R * K) == d[("bits_per_elem", "block32_8bit_scale")]
    assert np.floor((1 - 4.25 / 8) * 1000) / 10 == d[("saving_vs_fp8_percent", "block32")]
    for key, gb in [(k, v) for (kind, k), v in d.items() if kind == "footprint_gb"]:
        params = int(float(key))
        assert round(params * 4.5 / 8 / 1e9, 1) == gb


# ------------------------------------------------------------------- P3: E8M0 scale
def test_e8m0_decode_is_pure_power_of_two():
    e = np.arange(0, 255)
    v = O.e8m0_decode(e)
    m, ex = np.frexp(v)
    assert np.all(m == 0.5) and np.array_equal(ex - 1, e - 127)


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_scale_is_minimal_power_of_two(seed):
    rng = np.random.default_rng(seed)
    # block maxima spread over the whole exponent range, plus boundaries 6*2^k and +-1 ulp
    mags = np.float32(np.exp2(rng.uniform(-40, 126, size=3000)))
    k = np.arange(-35, 126)
    b = (6.0 * np.exp2(k.astype(np.float64))).astype(np.float32)
    mags = np.concatenate([mags, b, np.nextafter(b, np.float32(0)), np.nextafter(b, np.float32(np.inf)),
                           np.float32([0.0, 1e-45, 1e-8, 6e-9, 1.1e-8])])
    mags = mags[np.isfinite(mags)]
    e = O.mx_block_exponent(mags.astype(np.float64))
    for m, ee in zip(mags[::7], e[::7]):          # brute force on a subset
        assert bf_block_exponent(Fraction(float(m))) == ee
    mm = np.maximum(mags.astype(np.float64), float(np.float32(1e-8)))
    assert np.all(mm <= 6 * np.exp2(e.astype(np.float64)))
    assert np.all(mm > 6 * np.exp2((e - 1).astype(np.float64)))
    assert e.min() >= -29


# --------------------------------------------------------- P4: brute force, tiny
def _special_values():
    vals = [0.0, -0.0, 1e-45, -1e-45, 1e-39, 6.0, -6.0, 5.0, 3.5, 0.25, 0.75, 1.25, 1.75, 2.5]
    out = []
    for t in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]:
        for j in (-3, 0, 4):
            c = np.float32(t * 2.0 ** j)
            out += [c, np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(np.inf))]
    return np.float32(vals + out)


@pytest.mark.parametrize("block", [1, 2, 3, 4])
def test_mxfp4_bruteforce_tiny_blocks(block):
    rng = np.random.default_rng(100 + block)
    spec = _special_values()
    for trial in range(300):
        if trial % 2:
            xs = rng.choice(spec, size=block)
        else:
            xs = (rng.standard_normal(block) * np.exp2(rng.integers(-20, 20))).astype(np.float32)
        # put the block inside an MXFP4 block of 32 (rest zeros) -> same result
        x = np.zeros((1, 32), np.float32)
        x[0, :block] = xs
        codes, scales = O.mxfp4_quantize(x)
        c = O.unpack_codes(codes)[0]
        ref_c, ref_s = bf_mxfp4_block(list(x[0]))
        assert scales[0, 0] == ref_s
        assert list(c) == ref_c, (xs, list(c), ref_c)


def bf_nvfp4(x):
    """Brute force NVFP4 of a tiny [R, K] tensor with exact rationals.
    The per-tensor scale is the correctly rounded fp32 of amax / 2688 (checked
    here from its definition, not taken from the oracle)."""
    a = max(abs(Fraction(float(v))) for v in x.ravel())
    g = Fraction(float(np.float32(float(a)) / np.float32(2688.0))) if a else Fraction(1)
    # g must be the fp32 value nearest to a / 2688
    if a:
        gf = np.float32(float(g))
        exact = a / 2688
        lo, hi = np.nextafter(gf, np.float32(0)), np.nextafter(gf, np.float32(np.inf))
        assert abs(Fraction(float(gf)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(gf)) - exact) <= abs(Fraction(float(hi)) - exact)
    R, K = x.shape
    codes = np.zeros((R, K), np.uint8)
    sbytes = np.zeros((R, K // 16), np.uint8)
    for r in range(R):
        for b in range(K // 16):
            blk = x[r, b * 16:(b + 1) * 16]
            m = max(abs(Fraction(float(v))) for v in blk)
            sc = bf_nearest_e4m3(m / (6 * g))
            sbytes[r, b] = sc
            unit = E4M3_FR[sc] * g
            for j, v in enumerate(blk):
                mag = abs(Fraction(float(v)))
                if unit == 0:
                    c = 0
                else:
                    c = bf_nearest_e2m1(mag / unit)
                if np.signbit(v):
                    c |= 8
                codes[r, b * 16 + j] = c
    return codes, sbytes, g


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nvfp4_bruteforce_tiny(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 32)) * 0.5).astype(np.float32)
    x[0, 3] = 40.0                               # tensor max
    x[1, :16] = _special_values()[:16] * np.float32(1e-3)   # tiny block, sign of zero
    x[2, 16:] *= np.float32(1e-6)                # block scale deep in E4M3 subnormals / zero
    codes, sbytes, g = O.nvfp4_quantize(x)
    rc, rs, rg = bf_nvfp4(x)
    assert Fraction(float(g)) == rg
    assert np.array_equal(sbytes, rs)
    assert np.array_equal(O.unpack_codes(codes), rc)
    # saturation happens: some |x|/(s g) > 6 exist only when s rounded down
    assert sbytes.max() <= 0x7E


# --------------------------------------------------------- P5: exhaustive bf16
def test_exhaustive_bf16_elements_bruteforce():
    """Every finite bf16 bit pattern appears as an element, in a block where it
    is the maximum and in one anchored block (anchor 6*2^e sets the scale so
    the element lands in a chosen rounding region); oracle vs exact brute force
    with integer arithmetic."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    n = vals.size
    d = np.arange(n) % 6 - 1                     # region selector, -1..4
    mag = np.abs(vals).astype(np.float64)
    fl = np.floor(np.log2(np.where(mag > 0, mag, 1.0))).astype(np.int64)
    e_anchor = np.clip(fl + d, -29, 125)
    anchor = (6.0 * np.exp2(e_anchor.astype(np.float64))).astype(np.float32)
    x = np.zeros((n, 64), np.float32)
    x[:, 0] = vals          # block 0: the element alone (it is the max)
    x[:, 32] = vals         # block 1: element + anchor
    x[:, 33] = anchor
    codes, scales = O.mxfp4_quantize(x)
    c = O.unpack_codes(codes)
    # brute force with Python integers: v = |x| / 2^e is compared exactly with
    # the states via numerator/denominator arithmetic.
    for col, sc_col in ((0, 0), (32, 1)):
        for i in range(0, n, 1):
            xv = float(x[i, col])
            m = max(abs(Fraction(xv)), abs(Fraction(float(x[i, 33]))) if col == 32 else Fraction(0))
            e = int(scales[i, sc_col]) - 127
            if i % 97 == 0:                      # scale rule by brute force on a subset
                assert bf_block_exponent(m) == e
            v = abs(Fraction(xv)) / Fraction(2) ** e
            ref = bf_nearest_e2m1(v) | (8 if np.signbit(x[i, col]) else 0)
            assert c[i, col] == ref, (xv, e, c[i, col], ref)


# -------------------------------------------------- P6: outlier containment
@pytest.mark.parametrize("block", [32, 16])
def test_outlier_changes_only_its_block(block):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    c0, s0 = O.mxfp4_quantize(x, block=block)
    for (r, k) in [(0, 14), (2, 100), (3, 255)]:
        y = x.copy()
        y[r, k] = np.float32(50.0) * np.abs(x[r]).max()     # an outlier 50x the row's maximum
        c1, s1 = O.mxfp4_quantize(y, block=block)
        ch_s = np.argwhere(s0 != s1)
        assert ch_s.tolist() == [[r, k // block]]
        u0, u1 = O.unpack_codes(c0), O.unpack_codes(c1)
        ch_c = np.argwhere(u0 != u1)
        assert len(ch_c) > 0 and np.all(ch_c[:, 0] == r) and np.all(ch_c[:, 1] // block == k // block)


def test_nvfp4_outlier_contained_at_fixed_global_scale():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 128)).astype(np.float32)
    g = np.float32(0.01)
    c0, s0, _ = O.nvfp4_quantize(x, global_scale=g)
    y = x.copy()
    y[1, 37] = np.float32(50.0) * np.abs(x[1]).max()
    c1, s1, _ = O.nvfp4_quantize(y, global_scale=g)
    assert np.argwhere(s0 != s1).tolist() == [[1, 2]]
    ch = np.argwhere(O.unpack_codes(c0) != O.unpack_codes(c1))
    assert np.all(ch[:, 0] == 1) and np.all(ch[:, 1] // 16 == 2)


# ------------------------------------------------------------ P7: invariants
def test_mx_sign_symmetry_and_power_of_two_equivariance():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 128)) * 3).astype(np.float32)
    c, s = O.mxfp4_quantize(x)
    cn, sn = O.mxfp4_quantize(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(O.unpack_codes(c) ^ 8, O.unpack_codes(cn))
    for j in (-5, 3, 17):
        cj, sj = O.mxfp4_quantize((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(cj, c)
        assert np.array_equal(sj.astype(int), s.astype(int) + j)


def test_mx_dequant_quant_idempotent():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((16, 256)) * np.exp2(rng.integers(-10, 10, size=(16, 1)))).astype(np.float32)
    c, s = O.mxfp4_quantize(x)
    xh = O.dequantize("mxfp4", c, s)
    c2, s2 = O.mxfp4_quantize(xh)
    assert np.array_equal(O.dequantize("mxfp4", c2, s2), xh)


def test_mx_every_block_max_round_trip():
    """For every possible quantized block maximum (each state times each
    scale in range), quantizing the dequantized block reproduces it."""
    for e in range(-29, 126, 7):
        for i in range(1, 8):
            blk = np.zeros((1, 32), np.float32)
            blk[0, 0] = np.float32(O.E2M1_POSITIVE[i] * 2.0 ** e)
            blk[0, 1:8] = np.float32(np.array(O.E2M1_POSITIVE[:7]) * 2.0 ** e)
            c, s = O.mxfp4_quantize(blk)
            assert np.array_equal(O.dequantize("mxfp4", c, s), blk)


# --------------------------------- P8: the pages' scale equation and their demo
def equation_block_exponent(m: float) -> int:
    """Exponent of S_block = 2^ceil(log2(max / (6 S_global))) ("NVFP4
    Architecture", section "1. The Dual-Level Mathematical Formulation"), with
    S_global = 1 and the maximum first raised to 1e-8 as the emulation of
    section "End-to-End Implementation" does, evaluated in double precision
    (for an fp32 maximum, max / 6 in double is exact or rounds far from a
    power of two, so the ceiling is the exact one)."""
    return math.ceil(math.log2(max(m, float(np.float32(1e-8))) / 6.0))


@pytest.mark.parametrize("block", [32, 16])
def test_scale_equation_and_nearest_state_on_gaussian_fp32(block):
    """Gaussian fp32 blocks (one outlier column x40): every scale byte is the
    printed scale equation's exponent + 127 and every code the brute-force
    nearest state of x / S_block (exact rationals, sign copied)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((24, 512)) * 0.7).astype(np.float32)
    x[:, 5] *= 40
    c, s = O.mxfp4_quantize(x, block=block)
    codes = O.unpack_codes(c)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // block):
            blk = x[r, b * block:(b + 1) * block]
            e = equation_block_exponent(float(np.abs(blk).max()))
            assert int(s[r, b]) == e + 127
            for j, v in enumerate(blk):
                q = bf_nearest_e2m1(abs(Fraction(float(v))) / Fraction(2) ** e)
                assert codes[r, b * block + j] == q | (8 if np.signbit(v) else 0)


def test_page_demo_block_beats_naive():
    """The emulation demo's setting ("End-to-End Implementation"): 1024 values
    ~N(0, 0.5^2) with two outliers of about 25 and -31 planted, blocks of 16
    with power-of-two scales against one per-tensor scale.  The page prints no
    numbers, only that the block form reconstructs better; here the SNR gap
    is larger than 10 dB, and there is one scale per 16 elements."""
    rng = np.random.default_rng(2024)
    x = (rng.standard_normal(1024) * 0.5).astype(np.float32)
    x[100], x[700] = np.float32(24.5), np.float32(-31.2)
    xn = x.reshape(1, -1)
    c, s = O.mxfp4_quantize(xn, block=16)
    snr_block = O.reconstruction_snr_db(xn, O.dequantize("mxfp4", c, s))
    snr_naive = O.reconstruction_snr_db(x, O.naive_per_tensor_fp4(x))
    assert snr_block > snr_naive + 10
    assert s.shape == (1, 64)


def test_naive_per_tensor_worked_example():
    rows = _rows("naive_outlier_example.txt")
    x = np.array([float(r[0]) for r in rows])
    q_ref = np.array([float(r[1]) for r in rows])
    rec = O.naive_per_tensor_fp4(x)
    s = np.abs(x).max() / 6.0
    assert np.allclose(rec / s, q_ref, atol=0)
    # contrast: MXFP4 keeps resolution outside the outlier's block
    blk = np.zeros((1, 64), np.float32)
    blk[0, :6] = np.float32(x)
    blk[0, 40:46] = np.float32(x[[0, 1, 2, 4, 5, 0]])
    c, sc = O.mxfp4_quantize(blk)
    rec_mx = O.dequantize("mxfp4", c, sc)[0]
    assert np.all(rec_mx[40:46] != 0)


# ------------------------------------------------------- P9: E4M3 codec
def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = O.e4m3_decode(np.arange(256))
    same = (b == o) | (np.isnan(b) & np.isnan(o))
    assert np.all(same)


def test_e4m3_encode_matches_torch_cast():
    # dense sweep of fp32 values between 2^-12 and 464 (below the NaN overflow)
    bits = np.arange(np.float32(2.0 ** -12).view(np.uint32), np.float32(460.0).view(np.uint32), 4099,
                     dtype=np.uint32)
    v = bits.view(np.float32)
    mids = np.array([(O.e4m3_value_from_bits(c) + O.e4m3_value_from_bits(c + 1)) / 2 for c in range(0x7E)],
                    dtype=np.float32)
    v = np.concatenate([v, mids, np.float32([0.0, 448.0, 449.0, 2.0 ** -10, 2.0 ** -9])])
    ref = torch.from_numpy(np.minimum(v, 448.0).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_nearest_code(v.astype(np.float64), np.ones(v.shape))
    assert np.array_equal(got, ref)


def test_nvfp4_global_scale_self_consistency():
    """Parity unpinned reading, checked for consistency: the block holding the
    tensor maximum gets scale 448 and dequantized values stay within the
    E2M1 half-step of the input."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    x[4, 77] = 3.0
    c, s, g = O.nvfp4_quantize(x)
    assert g == np.float32(3.0) / np.float32(2688.0)
    assert s[4, 77 // 16] == 0x7E
    xh = O.dequantize("nvfp4", c, s, g)
    unit = np.repeat(O.e4m3_decode(s), 16, axis=1) * float(g)
    assert np.all(np.abs(xh - x) <= unit * 1.0 + 1e-12)


# ------------------------------------------------ P10/P11: products
def test_gemm_unit_scales_is_integer_gemm():
    rng = np.random.default_rng(12)
    M, N, K = 16, 24, 256
    ca = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    cb = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    a = O.dequantize("mxfp4", ca, ones_a)
    b = O.dequantize("mxfp4", cb, ones_b)
    y = O.gemm(a, b)
    ia = (2 * O.e2m1_decode(O.unpack_codes(ca))).astype(np.int64)   # 2q is an integer
    ib = (2 * O.e2m1_decode(O.unpack_codes(cb))).astype(np.int64)
    exact = (ia @ ib.T)
    assert np.array_equal(y.astype(np.float64) * 4, exact.astype(np.float64))


def _exact_dot_rows(a, b):
    return [[sum(Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(a.shape[1]))
             for n in range(b.shape[0])] for m in range(a.shape[0])]


def test_gemm_with_scales_bruteforce():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    ca, sa = O.mxfp4_quantize(x)
    cb, sb = O.mxfp4_quantize(w)
    a = O.dequantize("mxfp4", ca, sa)
    b = O.dequantize("mxfp4", cb, sb)
    y = O.gemm(a, b)
    ex = _exact_dot_rows(a, b)
    for m in range(3):
        for n in range(5):
            assert y[m, n] == np.float32(float(ex[m][n]))   # one rounding of the exact sum
    yb = O.gemm(a, b, out="bf16")
    ref_bf = torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(yb, ref_bf)


def test_dequant_values_bruteforce():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((2, 32)).astype(np.float32)
    c, s, g = O.nvfp4_quantize(x)
    xh = O.dequantize("nvfp4", c, s, g)
    codes = O.unpack_codes(c)
    for r in range(2):
        for k in range(32):
            q = E2M1_FR[codes[r, k] & 7] * (-1 if codes[r, k] & 8 else 1)
            exact = q * E4M3_FR[s[r, k // 16]] * Fraction(float(g))
            assert xh[r, k] == np.float32(float(exact))
    cm, sm = O.mxfp4_quantize(x)
    xm = O.dequantize("mxfp4", cm, sm)
    cu = O.unpack_codes(cm)
    for r in range(2):
        for k in range(32):
            q = E2M1_FR[cu[r, k] & 7] * (-1 if cu[r, k] & 8 else 1)
            assert Fraction(float(xm[r, k])) == q * Fraction(2) ** (int(sm[r, k // 32]) - 127)


def test_gemv_bruteforce():
    rng = np.random.default_rng(15)
    xb = torch.from_numpy(rng.standard_normal((2, 96)).astype(np.float32)).to(torch.bfloat16)
    xv = xb.to(torch.float32).numpy()
    w = (rng.standard_normal((7, 96)) * 0.02).astype(np.float32)
    cw, sw = O.mxfp4_quantize(w)
    y = O.gemv(xv, cw, sw)
    wh = O.dequantize("mxfp4", cw, sw)
    ex = _exact_dot_rows(xv, wh)
    for m in range(2):
        for n in range(7):
            f32 = np.float32(float(ex[m][n]))
            assert y[m, n] == torch.tensor(float(f32)).to(torch.bfloat16).item()


def test_grouped_equals_per_group_loop():
    rng = np.random.default_rng(16)
    G, N, K, T = 3, 8, 64, 11
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    offs = np.array([0, 4, 4, 11], np.int32)          # includes an empty expert
    wc = np.stack([O.mxfp4_quantize(w[g])[0] for g in range(G)])
    ws = np.stack([O.mxfp4_quantize(w[g])[1] for g in range(G)])
    y, ac, as_ = O.grouped_gemm(x, offs, wc, ws)
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        for r in range(r0, r1):
            c1, s1 = O.mxfp4_quantize(x[r:r + 1])
            assert np.array_equal(ac[r:r + 1], c1) and np.array_equal(as_[r:r + 1], s1)
            a = O.dequantize("mxfp4", c1, s1)
            b = O.dequantize("mxfp4", wc[g], ws[g])
            ex = _exact_dot_rows(a, b)
            for n in range(N):
                f32 = np.float32(float(ex[0][n]))
                assert y[r, n] == torch.tensor(float(f32)).to(torch.bfloat16).item()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 0x7F000000, size=200000, dtype=np.uint32)
    bits[:3] = [0x3F808000, 0x3F818000, 0x3F80FFFF]   # ties to even and just below
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.round_to_bf16(v), ref)


def test_tolerance_covers_bf16_rounding():
    a = np.ones((1, 4))
    b = np.ones((1, 4))
    y = np.array([[3.0]], np.float32)
    tol = O.gemm_tolerance(a, b, y, out="bf16")
    assert np.isclose(tol[0, 0], 4e-5 + 2.0 ** -6)


# ------------------------------------------------------ routed expert layers
def test_moe_route_is_a_stable_sort_by_expert():
    """The oracle's per-expert scan against Python's sort of (expert, flat
    index) keys; invalid ids (outside [0, experts)) are dropped."""
    rng = np.random.default_rng(31)
    for T, k, G in [(0, 2, 3), (1, 1, 1), (7, 2, 4), (40, 3, 5), (25, 2, 8)]:
        ids = rng.integers(-1, G + 1, size=(T, k)).astype(np.int32)   # includes -1 and G (invalid)
        offs, dest, src = O.moe_route(ids, G)
        keys = sorted((int(e), p) for p, e in enumerate(ids.reshape(-1)) if 0 <= e < G)
        want_dest = np.full(T * k, -1)
        for r, (e, p) in enumerate(keys):
            want_dest[p] = r
        assert np.array_equal(dest, want_dest)
        assert np.array_equal(src, [p // k for _, p in keys])
        assert offs[0] == 0 and offs[-1] == len(keys) and np.all(np.diff(offs) >= 0)
        for g in range(G):
            assert offs[g + 1] - offs[g] == sum(1 for e, _ in keys if e == g)


def test_moe_forward_equals_direct_per_token_sum():
    """Route + sorted grouped product + combine against the definition taken
    token by token: out[t] = sum_s w[t,s] * (Q(x_t) . W_hat_{e(t,s)}^T), with
    exact rational dot products (y kept in fp32 on the oracle side)."""
    rng = np.random.default_rng(32)
    T, K, N, G, k = 5, 64, 3, 3, 2
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    ids = np.array([[0, 2], [2, 1], [1, 1], [-1, 0], [2, 0]], np.int32)   # a repeated and an invalid slot
    tw = rng.random((T, k)).astype(np.float32)
    wc = np.stack([O.mxfp4_quantize(w[g])[0] for g in range(G)])
    ws = np.stack([O.mxfp4_quantize(w[g])[1] for g in range(G)])
    out, inter = O.moe_forward(x, ids, tw, wc, ws, y_out="f32", out="f32")
    for t in range(T):
        c, s = O.mxfp4_quantize(x[t:t + 1])
        a = O.dequantize("mxfp4", c, s)
        for n in range(N):
            exact = Fraction(0)
            bound = Fraction(0)
            for j in range(k):
                e = int(ids[t, j])
                if not 0 <= e < G:
                    continue
                b = O.dequantize("mxfp4", wc[e][n:n + 1], ws[e][n:n + 1])
                d = _exact_dot_rows(a, b)[0][0]
                exact += Fraction(float(tw[t, j])) * d
                bound += abs(Fraction(float(tw[t, j]))) * (abs(d) + 1)
            # y rounded to fp32, the combine rounded to fp32: two fp32 roundings
            assert abs(Fraction(float(out[t, n])) - exact) <= bound * Fraction(1, 2 ** 22)


# ------------------------------------------------------- fused RMSNorm + FP4
def test_rmsnorm_values_match_torch_rms_norm_fp64():
    """The oracle's RMSNorm against torch.nn.functional.rms_norm (a library
    routine) in float64."""
    rng = np.random.default_rng(41)
    for K in (32, 256, 8192 + 64, 14336):
        x = torch.from_numpy((rng.standard_normal((3, K)) * rng.uniform(0.1, 40, (3, 1))).astype(np.float32)).to(
            torch.bfloat16).float().numpy()
        gamma = rng.uniform(-0.5, 2.0, K).astype(np.float32)
        y = O.rmsnorm_values(x, gamma, 1e-6)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (K,), torch.from_numpy(gamma).double(),
                                           eps=1e-6).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_rmsnorm_closed_forms():
    # a constant row c: y = c / sqrt(c^2 + eps) * gamma
    K = 512
    x = np.full((2, K), 0.75, np.float32)
    x[1] = -3.0
    gamma = np.linspace(0.5, 1.5, K).astype(np.float32)
    y = O.rmsnorm_values(x, gamma, 0.0)
    assert np.allclose(y, np.sign(x) * gamma.astype(np.float64), rtol=1e-15, atol=0)
    eps = 0.25
    y = O.rmsnorm_values(x, np.ones(K, np.float32), eps)
    assert np.allclose(y[0], 0.75 / np.sqrt(0.75 ** 2 + eps), rtol=1e-15)
    # with eps = 0 and gamma = 1 the mean square of every row is 1, and scaling
    # a row does not change it
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 1000)).astype(np.float32)
    y = O.rmsnorm_values(x, np.ones(1000, np.float32), 0.0)
    assert np.allclose((y * y).mean(axis=1), 1.0, rtol=1e-14)
    assert np.allclose(O.rmsnorm_values(x * np.float32(64.0), np.ones(1000, np.float32), 0.0), y, rtol=1e-14)
    # zero row: y = 0 with x's sign; codes are signed zeros, scale byte 98
    z = np.zeros((1, 64), np.float32)
    z[0, 5] = -0.0
    c, s = O.rmsnorm_quantize(z, np.ones(64, np.float32), 1e-5)
    assert np.all(O.unpack_codes(c)[0, [i for i in range(64) if i != 5]] == 0)
    assert O.unpack_codes(c)[0, 5] == 8 and np.all(s == 98)


def test_rmsnorm_quantize_is_quantize_of_values():
    rng = np.random.default_rng(42)
    x = torch.from_numpy(rng.standard_normal((4, 1024)).astype(np.float32) * 5).to(torch.bfloat16).float().numpy()
    gamma = rng.uniform(-2, 2, 1024).astype(np.float32)
    y = O.rmsnorm_values(x, gamma, 1e-6).astype(np.float32)
    c1, s1 = O.rmsnorm_quantize(x, gamma, 1e-6)
    c2, s2 = O.mxfp4_quantize(y)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    g = np.float32(0.01)
    c3, s3 = O.rmsnorm_quantize(x, gamma, 1e-6, "nvfp4", global_scale=g)
    c4, s4, _ = O.nvfp4_quantize(y, global_scale=g)
    assert np.array_equal(c3, c4) and np.array_equal(s3, s4)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_rmsnorm_fragile_marks_exactly_the_decisions_a_perturbation_moves(fmt):
    """Planted near-boundary values are flagged; perturbing every value by a
    relative amount within the bound changes only flagged decisions."""
    rng = np.random.default_rng(5)
    g = np.float32(0.01) if fmt == "nvfp4" else None
    y = rng.standard_normal((64, 256)) * 2.0
    rel = 2.0 ** -17
    if fmt == "mxfp4":
        # a block maximum exactly at 6 * 2^0 and an element at a state midpoint
        y[0, :32] = np.clip(y[0, :32], -5.9, 5.9)
        y[0, 3] = 6.0
        y[1, :32] = np.clip(y[1, :32], -3.9, 3.9)
        y[1, 0], y[1, 7] = 4.0, 1.25
    block, elem = O.rmsnorm_fragile(y, rel, fmt, g)
    if fmt == "mxfp4":
        assert block[0, 0] and not block[1, 0] and elem[1, 7]
    for trial in range(4):
        yp = (y * (1.0 + rel * rng.uniform(-1, 1, y.shape))).astype(np.float32)
        c0, s0 = (O.mxfp4_quantize(y.astype(np.float32)) if fmt == "mxfp4"
                  else O.nvfp4_quantize(y.astype(np.float32), global_scale=g)[:2])
        c1, s1 = (O.mxfp4_quantize(yp) if fmt == "mxfp4" else O.nvfp4_quantize(yp, global_scale=g)[:2])
        assert np.all((s0 == s1) | block)
        k = 32 if fmt == "mxfp4" else 16
        ok = ~(np.repeat(block, k, axis=1) | elem)
        assert np.all((O.unpack_codes(c0) == O.unpack_codes(c1)) | ~ok)


# ------------------------------------------------ MXFP8 / MXFP6 element formats
# Closed-form value sets of the wider MX elements, written from the field
# definitions (sign, exponent with bias, mantissa; exponent field 0 subnormal).
def _closed_form_values(fmt):
    if fmt == "mxfp6_e2m3":        # bias 1: subnormals k/8, then steps 1/8, 1/4, 1/2
        return ([Fraction(k, 8) for k in range(16)] + [2 + Fraction(k, 4) for k in range(8)]
                + [4 + Fraction(k, 2) for k in range(8)])
    if fmt == "mxfp6_e3m2":        # bias 3: subnormals k/16, normals 2^(e-3)(1 + m/4)
        return [Fraction(k, 16) for k in range(4)] + [Fraction(2) ** (e - 3) * (1 + Fraction(m, 4))
                                                       for e in range(1, 8) for m in range(4)]
    raise KeyError(fmt)


@pytest.mark.parametrize("fmt", ["mxfp6_e2m3", "mxfp6_e3m2"])
def test_fp6_value_tables_closed_form(fmt):
    ref = _closed_form_values(fmt)
    got = O.element_positive_values(fmt)
    assert len(got) == 32 and [Fraction(float(v)) for v in got] == ref
    assert float(ref[-1]) == O.MX_ELEMENT_FORMATS[fmt][3]


@pytest.mark.parametrize("fmt,dt,n", [("mxfp8_e4m3", torch.float8_e4m3fn, 127),
                                      ("mxfp8_e5m2", torch.float8_e5m2, 124)])
def test_fp8_value_tables_match_torch(fmt, dt, n):
    codes = torch.arange(n, dtype=torch.uint8).view(dt).float().double().numpy()
    got = O.element_positive_values(fmt)
    assert len(got) == n and np.array_equal(got, codes)


def _bf_exponent(amax: Fraction, emax: Fraction) -> int:
    """Smallest integer e with amax <= emax * 2^e, by stepping."""
    e = 0
    while amax > emax * Fraction(2) ** e:
        e += 1
    while amax <= emax * Fraction(2) ** (e - 1):
        e -= 1
    return e


@pytest.mark.parametrize("fmt", ["mxfp8_e4m3", "mxfp8_e5m2", "mxfp6_e2m3", "mxfp6_e3m2", "mxfp4"])
def test_fmt_block_exponent_bruteforce(fmt):
    emax = Fraction(O.MX_ELEMENT_FORMATS[fmt][3])
    floor_amax = Fraction(float(np.float32(1e-8)))
    rng = np.random.default_rng(11)
    am = np.concatenate([np.exp2(rng.uniform(-40, 40, 300)).astype(np.float32),
                         np.float32(float(emax)) * np.exp2(np.arange(-5, 6)).astype(np.float32),
                         np.nextafter(np.float32(float(emax)), np.float32(np.inf)) * np.float32([1, 2, 0.5]),
                         np.float32([0.0, 1e-12, 1e-8])])
    got = O.mx_block_exponent_fmt(am, fmt)
    for a, e in zip(am, got):
        assert e == _bf_exponent(max(Fraction(float(a)), floor_amax), emax), (fmt, a)
    # the floor: -27 minus the exponent of Emax (the 1e-8 guard)
    p = int(np.floor(np.log2(float(emax))))
    assert O.mx_block_exponent_fmt(np.float32([0.0]), fmt)[0] == -27 - p


@pytest.mark.parametrize("fmt,dt", [("mxfp8_e4m3", torch.float8_e4m3fn), ("mxfp8_e5m2", torch.float8_e5m2)])
def test_fp8_quantize_matches_torch_cast(fmt, dt):
    """Elements: torch's round-to-nearest-even float8 cast of x / 2^e, with e
    from the brute-force exponent search."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 5] = -x[1, 5] * 1e4
    codes, scales = O.mx_quantize_fmt(x, fmt)
    emax = Fraction(O.MX_ELEMENT_FORMATS[fmt][3])
    fl = Fraction(float(np.float32(1e-8)))
    e = np.array([[_bf_exponent(max(Fraction(float(np.abs(b).max())), fl), emax) for b in row.reshape(-1, 32)]
                  for row in x])
    assert np.array_equal(scales, (e + 127).astype(np.uint8))
    scaled = (x.reshape(6, 4, 32).astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]).reshape(6, 128)
    ref = torch.from_numpy(scaled).float().to(dt).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def _bf_nearest_fr(v: Fraction, table) -> int:
    best, bd = None, None
    for i, t in enumerate(table):
        d = abs(v - t)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


@pytest.mark.parametrize("fmt", ["mxfp6_e2m3", "mxfp6_e3m2"])
def test_fp6_quantize_bruteforce(fmt):
    """Exact rational brute force over the closed-form table, including
    values placed exactly half-way between neighbouring states."""
    table = _closed_form_values(fmt)
    emax = table[-1]
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    x[0, :32] = np.float32([float(t) for t in table])                     # every state exactly
    mids = [(table[i] + table[i + 1]) / 2 for i in range(31)]
    x[1, :31] = np.float32([float(m) for m in mids]) * np.where(np.arange(31) % 2, -1, 1)
    x[1, 31] = float(emax)
    codes, scales = O.mx_quantize_fmt(x, fmt)
    un = O.unpack_elements(codes, 6)
    fl = Fraction(float(np.float32(1e-8)))
    for r in range(4):
        for b in range(2):
            blk = [Fraction(float(v)) for v in x[r, 32 * b:32 * b + 32]]
            e = _bf_exponent(max(max(abs(v) for v in blk), fl), emax)
            assert scales[r, b] == e + 127
            for i, v in enumerate(blk):
                idx = _bf_nearest_fr(abs(v) / Fraction(2) ** e, table)
                sign = 1 if float(x[r, 32 * b + i]) < 0 or (v == 0 and np.signbit(x[r, 32 * b + i])) else 0
                assert un[r, 32 * b + i] == idx | (sign << 5), (r, b, i)


def test_fp6_packing_bitstream():
    """Element i of a row occupies bits [6i, 6i + 6) of the row read as one
    little-endian integer."""
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 64, (3, 64))
    packed = O.pack_elements(codes, 6)
    assert packed.shape == (3, 48)
    for r in range(3):
        big = int.from_bytes(bytes(packed[r]), "little")
        assert [(big >> (6 * i)) & 63 for i in range(64)] == list(codes[r])
    assert np.array_equal(O.unpack_elements(packed, 6), codes)


def test_fmt_mxfp4_equals_pinned_mxfp4():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((8, 256)) * np.exp2(rng.integers(-30, 30, (8, 1)))).astype(np.float32)
    x[2, :32] = 0.0
    x[3, 40] = 1e30
    c0, s0 = O.mxfp4_quantize(x)
    c1, s1 = O.mx_quantize_fmt(x, "mxfp4")
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("fmt", ["mxfp8_e4m3", "mxfp8_e5m2", "mxfp6_e2m3", "mxfp6_e3m2"])
def test_fmt_dequant_exact_and_idempotent(fmt):
    """value(code) * 2^(E-127) against the Fraction decode of the fields, and
    quantize(dequantize(q)) reproduces the reconstruction exactly."""
    E, M, bias, _ = O.MX_ELEMENT_FORMATS[fmt]
    bits = 1 + E + M
    rng = np.random.default_rng(13)
    x = rng.standard_normal((5, 96)).astype(np.float32) * 3
    codes, scales = O.mx_quantize_fmt(x, fmt)
    y = O.dequantize_fmt(fmt, codes, scales)
    un = O.unpack_elements(codes, bits)
    for r in range(5):
        for k in range(96):
            c = int(un[r, k])
            mag = c & ((1 << (bits - 1)) - 1)
            e, m = mag >> M, mag & ((1 << M) - 1)
            v = (Fraction(m, 2 ** M) * Fraction(2) ** (1 - bias) if e == 0
                 else (1 + Fraction(m, 2 ** M)) * Fraction(2) ** (e - bias))
            v = -v if c >> (bits - 1) else v
            assert Fraction(float(y[r, k])) == v * Fraction(2) ** (int(scales[r, k // 32]) - 127)
    # re-quantizing the reconstruction is lossless; a block whose max rounded
    # down onto Emax/2 may take the next smaller scale, never another one
    c2, s2 = O.mx_quantize_fmt(y, fmt)
    d = scales.astype(int) - s2.astype(int)
    assert set(np.unique(d)) <= {0, 1}
    assert np.array_equal(O.dequantize_fmt(fmt, c2, s2), y)
    assert np.array_equal(c2[d.repeat(96 * bits // 8 // 3, 1) == 0], codes[d.repeat(96 * bits // 8 // 3, 1) == 0])


# ------------------------------------------- emulation variants (k, rule, S_global, tails)
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8_e4m3", "mxfp6_e2m3"])
def test_variant_default_equals_pinned_quantizers(fmt):
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-10, 10, (6, 1)))).astype(np.float32)
    x[0, 3] *= 300
    c, s = O.mx_quantize_variant(x, fmt, 32, "ceil")
    c2, s2 = O.mx_quantize_fmt(x, fmt)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    if fmt == "mxfp4":   # the emulation's default block of 16 (pinned against the page emulation)
        c, s = O.mx_quantize_variant(x, fmt, 16, "ceil")
        c2, s2 = O.mxfp4_quantize(x, block=16)
        assert np.array_equal(c, c2) and np.array_equal(s, s2)


def _bf_floor_exponent(m: Fraction) -> int:
    e = 0
    while Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    return e


@pytest.mark.parametrize("block", [16, 32])
def test_floor_rule_bruteforce_e2m1(block):
    """OCP rule: e = floor(log2 max|x|) - 2, elements nearest with saturation at 6."""
    rng = np.random.default_rng(block)
    x = (rng.standard_normal((4, 64)) * np.exp2(rng.integers(-8, 8, (4, 1)))).astype(np.float32)
    x[0, :block] = 0.0
    x[1, 2] = 7.5            # max with mantissa > 1.5: elements land in (6, 8) and saturate
    c, s = O.mx_quantize_variant(x, "mxfp4", block, "floor")
    codes = O.unpack_codes(c)
    fl = Fraction(float(np.float32(1e-8)))
    for r in range(4):
        for b in range(64 // block):
            blk = [Fraction(float(v)) for v in x[r, b * block:(b + 1) * block]]
            e = _bf_floor_exponent(max(max(abs(v) for v in blk), fl)) - 2
            assert s[r, b] == e + 127
            for i, v in enumerate(blk):
                idx = bf_nearest_e2m1(abs(v) / Fraction(2) ** e)
                sign = int(np.signbit(x[r, b * block + i]))
                assert codes[r, b * block + i] == idx | (sign << 3)


def test_floor_rule_e4m3_matches_saturating_torch_cast():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((5, 64)) * np.exp2(rng.integers(-12, 12, (5, 1)))).astype(np.float32)
    x[2, 9] = 500.0 * 2.0 ** 3      # max mantissa 1.95: elements up to 500 > 448 saturate
    c, s = O.mx_quantize_variant(x, "mxfp8_e4m3", 32, "floor")
    fl = Fraction(float(np.float32(1e-8)))
    e = np.array([[_bf_floor_exponent(max(Fraction(float(np.abs(b).max())), fl)) - 8 for b in row.reshape(-1, 32)]
                  for row in x])
    assert np.array_equal(s, (e + 127).astype(np.uint8))
    scaled = x.reshape(5, 2, 32).astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]
    scaled = np.clip(scaled, -448.0, 448.0).reshape(5, 64)
    ref = torch.from_numpy(scaled).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, ref)


def test_global_scale_bruteforce_k16():
    """S_block = 2^ceil(log2(m / (6 g))) with a per-tensor g: smallest e with
    m <= 6 g 2^e; elements nearest to x / (g 2^e)."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((3, 48)) * 5).astype(np.float32)
    g = np.float32(0.3712)
    c, s = O.mx_quantize_variant(x, "mxfp4", 16, "ceil", global_scale=g)
    codes = O.unpack_codes(c)
    G = Fraction(float(g))
    fl = Fraction(float(np.float32(1e-8)))
    for r in range(3):
        for b in range(3):
            blk = [Fraction(float(v)) for v in x[r, 16 * b:16 * b + 16]]
            m = max(max(abs(v) for v in blk), fl)
            e = 0
            while m > 6 * G * Fraction(2) ** e:
                e += 1
            while m <= 6 * G * Fraction(2) ** (e - 1):
                e -= 1
            assert s[r, b] == e + 127
            for i, v in enumerate(blk):
                idx = bf_nearest_e2m1(abs(v) / (G * Fraction(2) ** e))
                assert codes[r, 16 * b + i] == idx | (int(np.signbit(x[r, 16 * b + i])) << 3)
    y = O.dequantize_variant("mxfp4", c, s, 48, global_scale=g)
    q = O.dequantize("mxfp4", c, s)
    assert np.array_equal(y, (q * g).astype(np.float32))


@pytest.mark.parametrize("fmt,block,K", [("mxfp4", 32, 50), ("mxfp4", 16, 7), ("mxfp8_e5m2", 32, 33),
                                         ("mxfp6_e3m2", 32, 95)])
def test_zero_padded_tails_equal_explicit_padding(fmt, block, K):
    rng = np.random.default_rng(K)
    x = (rng.standard_normal((4, K)) * 4).astype(np.float32)
    c, s = O.mx_quantize_variant(x, fmt, block)
    Kp = -(-K // block) * block
    xp = np.zeros((4, Kp), np.float32)
    xp[:, :K] = x
    if block == 32:
        c2, s2 = O.mx_quantize_fmt(xp, fmt)
    else:
        c2, s2 = O.mxfp4_quantize(xp, block=block)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    y = O.dequantize_variant(fmt, c, s, K)
    assert y.shape == (4, K)


def test_naive_per_tensor_stored_form():
    """Codes of the stored form reproduce the pages' worked example, and its
    reconstruction equals naive_per_tensor_fp4 when fp32(max/6) is exact."""
    rows = _rows("naive_outlier_example.txt")
    x = np.array([[float(r[0]) for r in rows]], np.float32)
    x = np.concatenate([x, np.zeros((1, x.shape[1] % 2), np.float32)], axis=1) if x.shape[1] % 2 else x
    c, s = O.naive_per_tensor_quantize(x)
    q = O.e2m1_decode(O.unpack_codes(c))[0, :len(rows)]
    assert np.array_equal(q, np.array([float(r[1]) for r in rows]))
    rng = np.random.default_rng(2)
    y = (rng.standard_normal((3, 40)) * 2).astype(np.float32)
    y[1, 5] = 6.0 * 8.0                                  # max / 6 = 8 exactly
    c, s = O.naive_per_tensor_quantize(y)
    assert s == np.float32(8.0)
    assert np.array_equal(O.dequantize_naive(c, s).astype(np.float64), O.naive_per_tensor_fp4(y))


def test_snr_closed_form():
    assert abs(O.reconstruction_snr_db(np.array([1.0, 1.0]), np.array([1.0, 0.5])) - 10 * np.log10(8.0)) < 1e-12
    assert O.reconstruction_snr_db(np.array([2.0]), np.array([2.0])) == float("inf")
