"""mx_quantize_noalloc (static device scratch, no allocation) against
mx_quantize with a caller workspace: codes, scales and the per-tensor scale
must be identical.  Two calls in a row on one device, the second with a
smaller tensor (the scratch keeps the first call's partials), for every path
that uses the scratch (dynamic NVFP4, naive per-tensor FP4) and one that
does not (MXFP4)."""
import ctypes

import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_mx_amd as mx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _input(rows, cols, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rows // 3, cols // 5] = -300.0 * (seed + 1)      # the tensor maximum (negative)
    x[:, ::41] *= 30.0
    return torch.from_numpy(x).to(dtype).to(DEV)


def _noalloc(x, out, flags=0):
    d = out.desc()
    st = mx.lib().mx_quantize_noalloc(x.data_ptr(), mx._dt(x), x.stride(0), ctypes.byref(d), flags,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, mx.mx_status_string(st)


def _same(a, b, fmt):
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes), f"{fmt}: codes differ"
    if a.scales is not None:
        assert torch.equal(a.scales, b.scales), f"{fmt}: scales differ"
    if a.global_scale is not None:
        assert torch.equal(a.global_scale, b.global_scale), f"{fmt}: per-tensor scale differs"


@pytest.mark.parametrize("fmt", ["nvfp4", "fp4_tensor", "mxfp4"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry(fmt, dtype):
    # large first (many amax partials), then small (few partials): the second
    # call must not see the first call's partials
    for i, (rows, cols) in enumerate([(2050, 4096), (37, 256)]):
        announce(f"noalloc {fmt} {dtype} call {i} shape=({rows}, {cols})")
        x = _input(rows, cols, dtype, seed=i)
        ref = mx.mx_quantize(x, fmt)
        got = mx.empty_quantized(rows, cols, fmt, DEV)
        before = torch.cuda.memory_allocated()
        _noalloc(x, got)
        assert torch.cuda.memory_allocated() == before
        _same(got, ref, fmt)


def test_noalloc_static_global_and_errors():
    announce("noalloc nvfp4 static scale and argument errors")
    x = _input(64, 512, torch.float32, seed=5)
    ref = mx.mx_quantize(x, "nvfp4", static_global=0.004)
    got = mx.empty_quantized(64, 512, "nvfp4", DEV)
    got.global_scale.fill_(0.004)
    _noalloc(x, got, flags=mx.MX_QUANT_STATIC_GLOBAL)
    _same(got, ref, "nvfp4 static")
    # argument errors are reported as by mx_quantize (nothing enqueued)
    bad = mx.empty_quantized(64, 500, "nvfp4", DEV)
    d = bad.desc()
    assert mx.lib().mx_quantize_noalloc(x.data_ptr(), 0, 512, ctypes.byref(d), 0, None) == -5
    assert mx.lib().mx_quantize_noalloc(None, 0, 512, ctypes.byref(got.desc()), 0, None) == -1
