"""The GEMM acceptance bound and FP16 helpers shared by the tests.

The bound: ``max|C - C_ref| <= 5e-3 * max|C_ref| + ulp_fp16(max|C_ref|)``,
where ``C_ref`` is the oracle's float64-accumulated product.  The relative
part covers FP32 accumulation in any order and the FP16 rounding of both
outputs; the one-ulp part covers a result whose magnitude sits near zero.
The fused output stage (bias, activation) widens it as ``epilogue_bound``
states.
"""

from __future__ import annotations

import numpy as np

REL_TOL = 5e-3


def ulp_fp16(x: float) -> float:
    """Spacing of float16 values at magnitude ``x`` (``x`` finite)."""
    x = abs(float(x))
    h = np.float16(x)
    if not np.isfinite(h):
        h = np.float16(65504.0)
    return float(np.spacing(h))


def gemm_bound(C_ref) -> float:
    m = float(np.max(np.abs(np.asarray(C_ref, dtype=np.float64)))) if np.size(C_ref) else 0.0
    return REL_TOL * m + ulp_fp16(m)


def gemm_error(C, C_ref) -> float:
    C = np.asarray(C, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    if C.shape != C_ref.shape:
        raise AssertionError(f"shape {C.shape} != {C_ref.shape}")
    if not np.all(np.isfinite(C)):
        return float("inf")
    return float(np.max(np.abs(C - C_ref))) if C.size else 0.0


def assert_gemm_close(C, C_ref, what=""):
    err = gemm_error(C, C_ref)
    bound = gemm_bound(C_ref)
    assert err <= bound, f"{what}: max|C - C_ref| = {err:.4g} > bound {bound:.4g}"
    return err, bound


# The fused output stage, act(Z) with Z = sum + bias: the activations used
# (identity, ReLU, SiLU) change an error in Z by at most a factor of 1.1
# (SiLU's slope lies in about [-0.0998, 1.0998]), and the result is rounded
# to FP16 once more, half an ulp of the output.
ACT_LIPSCHITZ = 1.1


def epilogue_bound(Z_ref, Y_ref) -> float:
    my = float(np.max(np.abs(np.asarray(Y_ref, dtype=np.float64)))) if np.size(Y_ref) else 0.0
    return ACT_LIPSCHITZ * gemm_bound(Z_ref) + ulp_fp16(my)


def assert_epilogue_close(C, Z_ref, Y_ref, what=""):
    err = gemm_error(C, Y_ref)
    bound = epilogue_bound(Z_ref, Y_ref)
    assert err <= bound, f"{what}: max|C - act(Z_ref)| = {err:.4g} > bound {bound:.4g}"
    return err, bound


def ulp_bf16(x: float) -> float:
    """Spacing of BF16 values at magnitude ``x`` (normal range)."""
    x = abs(float(x))
    if x == 0:
        return 2.0 ** -133
    e = int(np.floor(np.log2(x)))
    return 2.0 ** (max(e, -126) - 7)


def bf16_bound(C_ref) -> float:
    """The GEMM bound with a BF16 output: 5e-3 max|C_ref| + one BF16 ulp."""
    m = float(np.max(np.abs(np.asarray(C_ref, dtype=np.float64)))) if np.size(C_ref) else 0.0
    return REL_TOL * m + ulp_bf16(m)
