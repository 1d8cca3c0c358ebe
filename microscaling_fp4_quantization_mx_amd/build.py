"""Build libmx.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Run as ``python -m microscaling_fp4_quantization_mx_amd.build``.  Every call
recompiles all sources.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmx.so")
# Measurement-only kernels of the benchmark (streaming read and copy ceilings),
# a library of their own so that libmx exports only the C ABI of include/mx.h.
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libmx_ceiling.so")
SOURCES = ["quantize.hip", "quantize_variant.hip", "gemm_mxfp4.hip", "gemm_nvfp4.hip", "gemm_mxw.hip", "gemm_fused.hip", "gemv.hip", "moe.hip",
           "norm_quant.hip", "noalloc.hip", "mx_api.cpp"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code (the compiler
# would otherwise form v_pk_* fp32 ops from scalar and float2 arithmetic).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Only the C entry points of include/mx.h are exported (mx_api.cpp marks them).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}", "-I",
          os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + lang + COMMON + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    cobj = _compile(CEILING_SRC)
    tmp = CEILING_LIB + ".tmp"
    r = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, cobj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
