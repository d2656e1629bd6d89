"""CPU oracle for the grouped NVFP4 W4A16 routed-MoE prefill path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct NumPy
implementation of what the path computes, written from the pages' statement of the
problem. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (``grouped_nvfp4_w4a16_amd``) never
imports, calls or links anything here, and this package shares no code with it.

Modules:
- ``codecs``: E2M1 / E4M3FN decode, FP32 -> BF16 round-to-nearest-even.
- ``moe``: dequant (exact and BF16-weight modes), align, grouped GEMM, SwiGLU clamp,
  combine, the whole routed layer, the router top-k, and the shared expert (a BF16
  SwiGLU MLP).

Every function is pinned by a ``-m "not gpu"`` test against something other than
itself (library routines, closed forms, brute force in exact rationals, worked
special cases). The one item with no such pin is listed below.

Parity unpinned: the error figures the pages print for their GB10 microtest
(max_abs 1.462067 / 0.998566 ..., forward_prefill_gemm module docs, section "What is
NOT bit-identical", error table). Their data distributions are not given, so those
numbers cannot be reproduced; only the structural fact that the grouped GEMM's error
against a BF16-weight reference is about half an output BF16 ulp is checked.
"""

from . import codecs, moe  # noqa: F401
