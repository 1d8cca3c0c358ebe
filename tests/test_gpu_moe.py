"""GPU parity of the routed expert layer (route -> gathered quantize -> grouped
W4A4 GEMM -> weighted combine) against the CPU oracle.  Routing outputs and
gathered codes/scales must match bit for bit; products within the GEMM
tolerance propagated through the combine."""
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


def bf16_values(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def ulp_bf16(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


@pytest.mark.parametrize("T,k,G,bad", [(0, 2, 4, 0), (1, 1, 1, 0), (37, 2, 4, 3), (1000, 2, 8, 10),
                                       (513, 4, 300, 5), (64, 1, 3, 64), (30000, 2, 8, 100),
                                       (600, 4, 1024, 20), (20, 2, 65536, 2), (4096, 2, 8, 0)])
def test_route_bit_exact(T, k, G, bad):
    """Stable expert order, including several chunks of pairs (2000 pairs and
    more), more experts than one counting workgroup's threads, and the largest
    expert count (a single chunk)."""
    announce(f"route T={T} topk={k} experts={G} invalid={bad}")
    rng = np.random.default_rng(T * 7 + G)
    ids = rng.integers(0, G, size=(T, k)).astype(np.int32)
    if bad:
        flat = ids.reshape(-1)
        pos = rng.choice(flat.size, size=min(bad, flat.size), replace=False)
        flat[pos] = rng.choice([-5, -1, G, G + 7], size=pos.size)
    offs, dest, src = mx.mx_moe_route(torch.from_numpy(ids).to(DEV), G)
    ro, rd, rs = O.moe_route(ids, G)
    assert np.array_equal(host(offs), ro)
    assert np.array_equal(host(dest), rd)
    assert np.array_equal(host(src)[: len(rs)], rs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_rows_bit_exact(dtype):
    announce(f"quantize_rows dtype={dtype}")
    rng = np.random.default_rng(5)
    X, K = 50, 320
    x = rng.standard_normal((X, K)).astype(np.float32)
    x[:, 3] *= 70
    if dtype == torch.bfloat16:
        x = bf16_values(x)
    idx = rng.integers(0, X, size=77).astype(np.int32)
    idx[[3, 20, 76]] = [-1, X, 1 << 30]                 # out of range -> zero rows
    xt = torch.from_numpy(x).to(dtype).to(DEV)
    q = mx.mx_quantize_rows(xt, torch.from_numpy(idx).to(DEV))
    xs = np.where(((idx >= 0) & (idx < X))[:, None], x[np.clip(idx, 0, X - 1)], 0.0).astype(np.float32)
    rc, rsc = O.mxfp4_quantize(xs)
    assert np.array_equal(host(q.codes), rc) and np.array_equal(host(q.scales), rsc)


@pytest.mark.parametrize("ydt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32)])
def test_combine(ydt, odt):
    announce(f"combine y={ydt} out={odt}")
    rng = np.random.default_rng(9)
    R, N, T, k = 90, 136, 40, 3
    y = rng.standard_normal((R, N)).astype(np.float32)
    if ydt == torch.bfloat16:
        y = bf16_values(y)
    dest = rng.integers(0, R, size=T * k).astype(np.int32)
    dest[[0, 5, 77]] = [-1, R, 1 << 29]
    w = rng.random(T * k).astype(np.float32)
    out = mx.mx_moe_combine(torch.from_numpy(y).to(ydt).to(DEV), torch.from_numpy(dest).to(DEV),
                            torch.from_numpy(w).to(DEV), T, k, out_dtype=odt)
    ref = O.moe_combine(y, dest, w, T, k).astype(np.float64)
    ok = (dest >= 0) & (dest < R)
    mag = np.zeros((T, N))
    for t in range(T):
        for s in range(k):
            p = t * k + s
            if ok[p]:
                mag[t] += abs(w[p]) * np.abs(y[dest[p]])
    tol = mag * 2.0 ** -21
    if odt == torch.bfloat16:
        ref = bf16_values(ref)
        tol = tol + ulp_bf16(ref)
    got = host(out.float()).astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()


def _expert_weights(G, N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)
    wq = mx.mx_quantize(torch.from_numpy(w).to(DEV))
    return wq, host(wq.codes).reshape(G, N, K // 2), host(wq.scales).reshape(G, N, K // 32)


def _combine_tolerance(ids, tw, dest, yref_rows, ytol_rows, out_ref):
    """|out_gpu - out_ref| <= sum_s |w_s| tol_y(row_s) + fp32 combine rounding
    + one bf16 ulp of out_ref."""
    T, k = ids.shape
    tol = np.zeros_like(out_ref, dtype=np.float64)
    for t in range(T):
        for s in range(k):
            r = dest[t * k + s]
            if r >= 0:
                tol[t] += abs(tw[t, s]) * (ytol_rows[r] + np.abs(yref_rows[r]) * 2.0 ** -21)
    return tol + ulp_bf16(out_ref)


@pytest.mark.parametrize("T,k,G", [(64, 2, 4), (33, 1, 3), (100, 3, 5)])
def test_moe_forward_small(T, k, G):
    announce(f"moe forward T={T} topk={k} experts={G}")
    N, K = 96, 288
    rng = np.random.default_rng(T + k)
    x = bf16_values(rng.standard_normal((T, K)).astype(np.float32) * 2)
    ids, tw = W.topk_routing(T, G, k, seed=T)
    ids[0, 0] = -1                                        # one dropped pair
    wq, wc, ws = _expert_weights(G, N, K, seed=G)
    out = mx.moe_forward(torch.from_numpy(x).to(torch.bfloat16).to(DEV), torch.from_numpy(ids).to(DEV),
                         torch.from_numpy(tw).to(DEV), wq, G, N)
    ref, inter = O.moe_forward(x, ids, tw, wc, ws)
    # tolerance of every routed row's product
    off = inter["offsets"]
    ytol = np.zeros_like(inter["y"], dtype=np.float64)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            ah = O.dequantize("mxfp4", inter["a_codes"][r0:r1], inter["a_scales"][r0:r1])
            ytol[r0:r1] = O.gemm_tolerance(ah, O.dequantize("mxfp4", wc[g], ws[g]), inter["y"][r0:r1], out="bf16")
    tol = _combine_tolerance(ids, tw, inter["dest_row"], inter["y"], ytol, ref)
    got = host(out.float()).astype(np.float64)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:3], np.abs(got - ref).max())


def test_moe_full_size_sampled():
    """The benchmark's routed layer (4096 tokens, top-2 of 8 experts, N=4096,
    K=14336) in its launch configuration: routing bit-exact, gathered codes of
    sampled rows bit-exact, sampled outputs within tolerance."""
    w = W.MOE
    T, G, N, K, k = w.M, w.experts, w.N, w.K, W.MOE_TOPK
    announce(f"moe full size T={T} topk={k} G={G} N={N} K={K}")
    d = W.make(w)
    ids, tw = W.topk_routing(T, G, k)
    wq = mx.mx_quantize(torch.from_numpy(d["w"].reshape(G * N, K)).to(DEV))
    xt = torch.from_numpy(d["x"]).to(torch.bfloat16).to(DEV)
    bufs = {}
    out = mx.moe_forward(xt, torch.from_numpy(ids).to(DEV), torch.from_numpy(tw).to(DEV), wq, G, N, bufs=bufs)
    offs, dest, src = mx.mx_moe_route(torch.from_numpy(ids).to(DEV), G)
    ro, rd, rs = O.moe_route(ids, G)
    assert np.array_equal(host(offs), ro) and np.array_equal(host(dest), rd)
    assert np.array_equal(host(src)[: len(rs)], rs)
    rng = np.random.default_rng(77)
    toks = rng.choice(T, size=12, replace=False)
    cols = np.sort(rng.choice(N, size=24, replace=False))
    got = host(out.float())[np.ix_(toks, cols)].astype(np.float64)
    wc_all, ws_all = host(wq.codes), host(wq.scales)
    ref = np.zeros((len(toks), len(cols)))
    tol = np.zeros_like(ref)
    for i, t in enumerate(toks):
        c, s = O.mxfp4_quantize(d["x"][t:t + 1])
        a = O.dequantize("mxfp4", c, s)
        for j in range(k):
            e = int(ids[t, j])
            rows = e * N + cols
            b = O.dequantize("mxfp4", wc_all[rows], ws_all[rows])
            yr = O.gemm(a, b, out="bf16")[0]
            yt = O.gemm_tolerance(a, b, yr[None, :], out="bf16")[0]
            ref[i] += float(tw[t, j]) * yr.astype(np.float64)
            tol[i] += abs(float(tw[t, j])) * (yt + np.abs(yr) * 2.0 ** -21)
    ref = bf16_values(ref.astype(np.float32)).astype(np.float64)
    tol += ulp_bf16(ref)
    assert np.all(np.abs(got - ref) <= tol), np.abs(got - ref).max()
