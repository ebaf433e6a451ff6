"""CPU oracle for the block-scaled GEMM family (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The product path (``fp4_gemm_moe_amd``) never imports it, and it
imports nothing from the product path: the two share no code.

Sources (the pages are cited by title and section):
  * HALOps "GEMM" API page: sections batch_gemm, dense_gemm,
    fused_swiglu_quant, group_contiguous_gemm, group_masked_gemm,
    group_wise_quant, prefill_permute_to_masked_gemm.
  * flashrt/fp4-gemm kernel page: function list and Notes (NVFP4 A4W4).
  * cuDNN Frontend "Grouped GEMM + dGLU (SM100)": Step 1 equation (the
    dequantize-dequantize definition of the block-scaled grouped GEMM) and
    the Data Types table (formats and scale-vector sizes).
  * The element formats themselves (E4M3, E2M1, UE8M0) are only named on the
    pages; their bit-level definitions follow the OCP Microscaling (MX) v1.0
    specification.

Modules:
  formats  - bit-level decode tables and round-to-nearest-even encoders
  quant    - MX (UE8M0 / 32) and NVFP4 (UE4M3 / 16 + FP32 global) quantisation
  gemm     - dense, batch, grouped-contiguous and grouped-masked scaled GEMMs
  swiglu   - SwiGLU followed by re-quantisation

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (exhaustive tables, brute force with exact rationals,
integer-exact GEMMs, closed forms, loop-of-dense identities).  The NVFP4
recipe has no worked values on the pages; its internal steps are pinned by
enumeration, but agreement with other NVFP4 implementations is "parity
unpinned".
"""

from . import formats, quant, gemm, swiglu  # noqa: F401
