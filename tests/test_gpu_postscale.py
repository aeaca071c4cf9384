"""Which product each kernel variant computes, for the FP16 formats 0 and 1.

Every streaming variant compiled for these formats, and the stream-K and
LDS tiles of 16 and 32 rows, apply the group scale to the FP32 sum of each
128-deep block: the result is the product with the exact weights
(q - z) * s, never rounded to FP16.  The larger tiles scale each weight in
FP16 first, as the oracle's definition does.  Both are within the GEMM bound
of the oracle; this test shows which one a variant computes.

With K in the thousands the two products round to different FP16 outputs
in about 40% of places, while FP32 accumulation moves an output across a
rounding boundary in only a few percent.  So a variant's outputs equal the
FP16 rounding of its own product in at least 95% of places, and the test
checks that the other product would not pass the same check.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs, make_inputs_awq
from tests.gpu_util import run_gemm, run_gemm_awq, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu

MIN_MATCH = 0.95      # outputs equal to the FP16 rounding of the variant's product
MAX_CROSS = 0.80      # the same check against the other product must fail


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _exact_weights(Bq, S, Z, group):
    """(q - z) * s in float64, with no rounding (z = 8 without zero points)."""
    q = oracle.unpack_codes(Bq).astype(np.float64)
    z = 8.0 if Z is None else np.repeat(np.asarray(Z, dtype=np.float64), group, axis=0)
    return (q - z) * np.repeat(np.asarray(S, dtype=np.float64), group, axis=0)


def _match(C, ref64):
    return float(np.mean(C.view(np.uint16) == ref64.astype(np.float16).view(np.uint16)))


# forced plan (mb, nb, wk, splits, depth[, tile]), the kernel it names, and
# whether that kernel applies the scale to the sums
PLANS = [("1,2,8,1,2", "gemm_kernel<1,2,8,2>", True),
         ("1,4,4,1,2", "gemm_kernel<1,4,4,2>", True),
         ("1,1,8,1,2", "gemm_kernel<1,1,8,2>", True),
         ("1,4,4,3,2", "gemm_kernel<1,4,4,2>", True),
         ("1,4,8,0,4,4", "gemm_sk_kernel<1,4,4,8>", True),
         ("2,4,8,0,3,4", "gemm_sk_kernel<2,4,3,8>", True),
         ("4,4,8,0,3,4", "gemm_sk_kernel<4,4,3,8>", False),
         ("1,2,8,1,4,2", "gemm_lds_kernel<1,2,1,8,4>", True),
         ("1,2,8,4,4,2", "gemm_lds_kernel<1,2,1,8,4>", True),
         ("2,2,8,1,4,2", "gemm_lds_kernel<2,2,1,8,4>", True),
         ("4,1,8,1,3,2", "gemm_lds_kernel<4,1,1,8,3>", False)]


@pytest.mark.parametrize("plan,kernel,post", PLANS)
@pytest.mark.parametrize("zp", [False, True])
def test_variant_product(plan, kernel, post, zp):
    M, K, N, group = 3, 4096, 512, 128
    if zp:
        A, Bq, S, Z = make_inputs_awq(M, K, N, group, seed=41)
    else:
        A, Bq, S = make_inputs(M, K, N, group, seed=41)
        Z = None
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, group)
    assert desc.startswith(kernel + " "), desc
    say("post-scale", plan, "zp" if zp else "f16", desc)
    C = run_gemm_awq(A, Bq, S, Z, group, 0) if zp else run_gemm(A, Bq, S, group)

    A64 = A.astype(np.float64)
    exact = A64 @ _exact_weights(Bq, S, Z, group)
    if zp:
        _, rounded = oracle.gemm_awq(A, Bq, S, Z, group, 0)
    else:
        _, rounded = oracle.gemm(A, Bq, S, group)
    assert_gemm_close(C, rounded, f"plan {plan}")
    m_exact, m_rounded = _match(C, exact), _match(C, rounded)
    say("  match exact-weight product", m_exact, "rounded-weight product", m_rounded)
    mine, other = (exact, rounded) if post else (rounded, exact)
    assert _match(C, mine) >= MIN_MATCH
    assert _match(other.astype(np.float16), mine) <= MAX_CROSS  # the check discriminates
    assert _match(C, other) <= MAX_CROSS
