"""Plain CPU oracle for the W4A16 matmul (test infrastructure only).

This package is test infrastructure.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and nothing here imports the product.

It is written from the pages' description of what the method computes, in
plain numpy, with no blocking, fusion or reordering beyond that description:

* "Quant Marlin kernel" explainer (aicassindra.com), section "The
  architecture: every piece explained", top row: eight 4-bit codes per 32-bit
  word, one FP16 scale per group of weights (commonly 128); middle row: codes
  become FP16 and are multiplied by the group scale, then enter an FP16 matrix
  multiply with FP32 (or FP16) accumulation; bottom rows: FP16 activations in,
  FP16 output out.
* Same page, "End-to-end flow": FP16 activations (tokens x in-features) times
  INT4 weights (in-features x out-features), per-128 group scales.

* Same page, "End-to-end flow": the product goes straight on to a bias add
  or an activation (``gemm_fused``).
* "Low-Precision Quantization Kernels in Production" (llms.blog), section 1
  and the table of section 5 (AWQ checkpoints), introduction and section 4
  (BF16): zero points and BF16 (``dequant_awq``, ``gemm_awq``); section 1
  and the same table (4-bit and 8-bit checkpoints): 8-bit weights
  (``dequant8``, ``gemm8``, ``repack8``).
* "The anthology of the SOTA" (dmarx.github.io), the MARLIN note, "Key
  results" (Figure 15, Sparse-MARLIN): the 2:4 sparse variant
  (``dequant_sparse24``, ``gemm_sparse24``, ``repack_sparse24``).

Readings where the pages leave a step open (zero point 8, LSB-first nibble
order along K, scale layout ``[K/group][N]``, single RNE rounding of the
dequantised weight, the bias and activation of the fused output) are stated
in ``w4a16_ref``'s docstrings.
"""

from .w4a16_ref import (  # noqa: F401
    ZERO_POINT,
    LAYOUT_VERSION,
    unpack_codes,
    pack_codes,
    dequant,
    gemm,
    gemm_f32,
    gemm_columns,
    repack,
    unrepack,
    ACT_NONE,
    ACT_RELU,
    ACT_SILU,
    activation,
    epilogue,
    gemm_fused,
    DTYPE_F16,
    DTYPE_BF16,
    bf16_to_f64,
    f64_to_bf16,
    dequant_awq,
    gemm_awq,
    ZERO_POINT8,
    unpack_codes8,
    pack_codes8,
    dequant8,
    gemm8,
    repack8,
    unrepack8,
    sparse24_keep,
    dequant_sparse24,
    gemm_sparse24,
    repack_sparse24,
)
