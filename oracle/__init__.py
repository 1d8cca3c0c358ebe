"""CPU oracle for block-scaled FP4 quantization and the products that consume it.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is the plain, slow,
fp64 reference that the HIP library is checked against.  Only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library and its Python binding never do, and the oracle never
imports them.  It shares no code, table or constant with the HIP path.

Sources (the pages are web pages; each function cites page title + section):
  * "NVFP4 Architecture: Microscaling & 4-Bit LLMs on Blackwell" -- E2M1 table,
    E8M0 scale, the dual-level scaling equations and the PyTorch emulation.
  * "How Microscaling FP4 (MXFP4) Halves Memory Bandwidth ..." -- 32-element
    MXFP4 blocks, E2M1 saturation at +-6.
  * "NVIDIA NVFP4 quantization" -- 16-element NVFP4 blocks with an 8-bit scale.
  * "MXFP4" (wiki card) -- OCP MXFP4: E8M0 scales, block size 32.

Parity unpinned: the NVFP4 per-tensor scale g = fp32(amax_tensor / (6*448))
and the choice of E4M3 round-to-nearest-even for the NVFP4 block scale have no
value printed on the pages; they are pinned only by self-consistency checks
(the largest block scale decodes to 448, round trips) and, for the E4M3 codec
itself, by torch's float8_e4m3fn.
"""
from .mx_oracle import *  # noqa: F401,F403
