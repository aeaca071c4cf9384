"""The streaming kernel with its activations staged in LDS (batches of at
most four rows whose rows over one workgroup's K range fit in 32 KiB, FP16
activations; the plan description then ends in ``activations=lds``).

The staged path must give the oracle's answer within the GEMM bound, be exact
on one-hot rows, and produce exactly the bits of the same kernel variant
reading its activations from global memory: only where the activations come
from differs, not one addition.  Edge cases: K ranges split unevenly between
workgroups, waves that own no K block (they still meet the workgroup
barrier), the size threshold on both sides, every dense weight format and the
fused output stage.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_bias, make_inputs, make_inputs_awq
from tests.gpu_util import run_gemm, run_gemm8, run_gemm_awq, run_gemm_fused, say
from tests.test_gpu_w8 import _words8
from tests.tolerance import assert_epilogue_close, assert_gemm_close, bf16_bound, gemm_bound

pytestmark = pytest.mark.gpu

STAGED = "activations=lds"


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


@pytest.mark.parametrize("M,K,N,group,staged", [
    (1, 128, 16, 128, True),       # one K block: three of four waves own none
    (2, 384, 208, 128, True),      # ragged column tile
    (3, 4096, 4096, 128, True),
    (4, 4096, 4096, 128, True),    # 32 KiB exactly: the largest staged size
    (4, 4224, 4096, 128, False),   # 33 KiB: activations from global memory
    (5, 4096, 4096, 128, False),   # five rows: activations from global memory
    (1, 11008, 4096, 128, True),
    (2, 11008, 4096, 128, False),
    (1, 4096, 12288, 4096, True),  # one scale group
    (2, 16384, 64, 128, True),     # split K: 128 K blocks in three unequal ranges
])
def test_staged_activations_match_oracle(M, K, N, group, staged):
    desc = w4.w4a16_describe(M, K, N, group)
    assert (STAGED in desc) == staged, desc
    A, Bq, S = make_inputs(M, K, N, group, seed=M * 7 + K + N)
    say("staged", M, K, N, group, desc)
    C = run_gemm(A, Bq, S, group)
    _, C64 = oracle.gemm(A, Bq, S, group)
    assert_gemm_close(C, C64, f"M={M} K={K} N={N} g={group}")


# Every streaming variant with one row block, unsplit and split so that the
# splits' K ranges differ in length (K = 3584: 28 K blocks) and some waves
# own no K block (seven splits of four blocks for four waves; five splits of
# five or six blocks for eight waves).
STAGED_PLANS = ["1,4,4,7,2", "1,1,8,1,2", "1,1,8,5,2", "1,2,8,1,2", "1,2,8,4,2",
                "1,4,4,1,2", "1,4,4,3,2", "1,4,4,1,4", "1,4,4,6,4"]


@pytest.mark.parametrize("plan", STAGED_PLANS)
@pytest.mark.parametrize("M", [1, 4])
def test_staged_forced_plans(plan, M):
    K, N, group = 3584, 208, 128
    A, Bq, S = make_inputs(M, K, N, group, seed=11 + M)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, group)
    mb, nb, wk, splits, depth = (int(x) for x in plan.split(","))
    assert desc.startswith(f"gemm_kernel<{mb},{nb},{wk},{depth}>"), desc
    assert f"splits={splits} " in desc and STAGED in desc, desc
    say("staged forced", plan, M, desc)
    C = run_gemm(A, Bq, S, group)
    _, C64 = oracle.gemm(A, Bq, S, group)
    assert_gemm_close(C, C64, f"plan {plan} M={M}")


@pytest.mark.parametrize("plan", ["1,1,8,1,2", "1,2,8,3,2", "1,4,4,2,4"])
def test_staged_rows_equal_global_rows(plan):
    """Rows 0..3 of a five-row product (activations from global memory) and
    the four-row product of the same rows (staged) with the same forced
    variant: every output row is the same sequence of operations, so the
    bits agree."""
    K, N, group = 2048, 272, 128
    A5, Bq, S = make_inputs(5, K, N, group, seed=23)
    w4.w4a16_set_forced_plan(plan)
    d4, d5 = w4.w4a16_describe(4, K, N, group), w4.w4a16_describe(5, K, N, group)
    assert STAGED in d4 and STAGED not in d5, (d4, d5)
    assert d4.split(" ")[0] == d5.split(" ")[0], (d4, d5)
    say("staged vs global", plan, d4)
    C4 = run_gemm(np.ascontiguousarray(A5[:4]), Bq, S, group)
    C5 = run_gemm(A5, Bq, S, group)
    assert np.array_equal(C4.view(np.uint16), C5[:4].view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(1, 384, 48), (2, 1024, 80), (4, 4096, 64)])
def test_staged_one_hot_rows_exact(M, K, N):
    """One nonzero activation per row, a power of two: each output is one
    weight times it, exact, so a fragment read from the wrong place in LDS
    cannot pass."""
    _, Bq, S = make_inputs(1, K, N, 128, seed=M + K)
    rng = np.random.default_rng(M + 3)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), rng.integers(0, K, size=M)] = (2.0 ** rng.integers(-2, 3, size=M)).astype(
        np.float16)
    assert STAGED in w4.w4a16_describe(M, K, N, 128)
    C = run_gemm(A, Bq, S, 128)
    C16, _ = oracle.gemm(A, Bq, S, 128)
    assert np.array_equal(C.astype(np.float64), C16.astype(np.float64))


@pytest.mark.parametrize("dtype,zp", [(0, True), (1, False), (1, True)])
@pytest.mark.parametrize("M,K,N", [(1, 3584, 208), (3, 1024, 80)])
def test_staged_zero_point_and_bf16_formats(dtype, zp, M, K, N):
    """FP16 with zero points stages its activations; the BF16 formats keep
    the global path (measured faster for them).  Both match the oracle."""
    A, Bq, S, Z = make_inputs_awq(M, K, N, 128, seed=M + N + dtype, bf16=dtype == 1)
    Z = Z if zp else None
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fmt = (2 if dtype else 0) + (1 if zp else 0)   # the w4a16_format number
    desc = w4.w4a16_plan_describe(M, K, N, 128, fmt, cus)
    assert (STAGED in desc) == (dtype == 0), desc
    say("staged awq", dtype, zp, M, K, N, desc)
    C = run_gemm_awq(A, Bq, S, Z, 128, dtype)
    _, C64 = oracle.gemm_awq(A, Bq, S, Z, 128, dtype)
    got = oracle.bf16_to_f64(C) if dtype else np.asarray(C, dtype=np.float64)
    bound = bf16_bound(C64) if dtype else gemm_bound(C64)
    err = float(np.max(np.abs(got - C64)))
    assert err <= bound, f"max|C - C_ref| = {err:.4g} > {bound:.4g}"


@pytest.mark.parametrize("M,K,N", [(1, 3584, 208), (4, 2048, 64)])
def test_staged_eight_bit_weights(M, K, N):
    A, _, S = make_inputs(M, K, N, 128, seed=M + N)
    Bq8 = _words8(K, N, M + 5)
    desc = w4.w8a16_describe(M, K, N, 128)
    assert STAGED in desc, desc
    say("staged w8", M, K, N, desc)
    C = run_gemm8(A, Bq8, S, 128)
    _, C64 = oracle.gemm8(A, Bq8, S, 128)
    assert_gemm_close(C, C64, f"w8 M={M} K={K} N={N}")


@pytest.mark.parametrize("plan", [None, "1,1,8,7,2", "1,4,4,3,4"])
@pytest.mark.parametrize("act", [w4.W4A16_ACT_NONE, w4.W4A16_ACT_SILU])
def test_staged_fused_epilogue(plan, act):
    M, K, N, group = 3, 3584, 208, 128
    A, Bq, S = make_inputs(M, K, N, group, seed=31)
    bias = make_bias(N, seed=32)
    w4.w4a16_set_forced_plan(plan)
    assert STAGED in w4.w4a16_describe(M, K, N, group)
    C = run_gemm_fused(A, Bq, S, group, bias, act)
    _, C64 = oracle.gemm(A, Bq, S, group)
    Z = oracle.epilogue(C64, bias, oracle.ACT_NONE)
    assert_epilogue_close(C, Z, oracle.activation(Z, act), f"plan {plan} act {act}")
