"""Parity of the fused output stage (w4a16_gemm_fused) with the oracle.

``C = act(A . dequant(B) + bias)`` must satisfy the epilogue bound of
``tests/tolerance.py`` against the oracle's float64 ``act(Z)``, through every
kernel family and split-K path; where the arithmetic leaves no rounding (no
bias and no activation; zero activations with a bias and ReLU) it must be
exact.
"""

from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_bias, make_inputs
from tests.gpu_util import dev, repack_on_device, run_gemm, run_gemm_fused, say
from tests.tolerance import assert_epilogue_close

pytestmark = pytest.mark.gpu

ACTS = {"none": w4.W4A16_ACT_NONE, "relu": w4.W4A16_ACT_RELU, "silu": w4.W4A16_ACT_SILU}


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


@functools.lru_cache(maxsize=None)
def _case(M, K, N, group, seed):
    A, Bq, S = make_inputs(M, K, N, group, seed=seed)
    bias = make_bias(N, seed=seed + 1)
    _, C64 = oracle.gemm(A, Bq, S, group)
    return A, Bq, S, bias, C64


def _check(C, C64, bias, act, what):
    Z = oracle.epilogue(C64, bias, oracle.ACT_NONE)
    Y = oracle.activation(Z, act)
    assert_epilogue_close(C, Z, Y, what)


# One variant of each kernel family, with and without split-K; M = 45 and
# N = 208 leave ragged row and column tiles.
FUSED_PLANS = ["1,2,8,1,2", "1,4,4,7,2", "1,4,4,3,4",                  # streaming kernel
               "4,1,8,1,3,2", "8,2,8,2,3,2", "1,2,8,1,4,2", "4,2,4,3,3,2,0,2",  # LDS kernel
               "2,4,8,0,3,4", "1,4,8,5,4,4"]                                  # stream-K kernel
KERNEL_OF_TILE = {0: "gemm_kernel", 2: "gemm_lds_kernel", 4: "gemm_sk_kernel"}


@pytest.mark.parametrize("plan", FUSED_PLANS)
@pytest.mark.parametrize("act,with_bias", [("none", True), ("relu", True), ("silu", True),
                                           ("silu", False), ("relu", False)])
def test_fused_forced_plans(monkeypatch, plan, act, with_bias):
    M, K, N, group = 45, 3584, 208, 128
    A, Bq, S, bias, C64 = _case(M, K, N, group, 5)
    b = bias if with_bias else None
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, group)
    fields = [int(x) for x in plan.split(",")]
    assert desc.startswith(KERNEL_OF_TILE[fields[5] if len(fields) > 5 else 0] + "<"), desc
    say("fused", plan, act, "bias" if with_bias else "no bias", desc)
    C = run_gemm_fused(A, Bq, S, group, b, ACTS[act])
    _check(C, C64, b, ACTS[act], f"plan {plan} act {act} bias {with_bias}")


@pytest.mark.parametrize("M,K,N,group", [(1, 4096, 4096, 128), (3, 256, 48, 128),
                                         (16, 1024, 272, 128), (33, 768, 80, 128),
                                         (128, 4096, 1024, 128), (300, 1280, 96, 1280),
                                         (513, 256, 64, 128), (8, 13824, 160, 13824)])
def test_fused_default_plans(M, K, N, group):
    """The plans the heuristic picks, SiLU with a bias."""
    A, Bq, S, bias, C64 = _case(M, K, N, group, M * 7 + K)
    say("fused default", M, K, N, group, w4.w4a16_describe(M, K, N, group))
    C = run_gemm_fused(A, Bq, S, group, bias, w4.W4A16_ACT_SILU)
    _check(C, C64, bias, oracle.ACT_SILU, f"M={M} K={K} N={N} g={group}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (16, 4096, 12288), (45, 3584, 208),
                                   (128, 4096, 4096), (600, 1024, 512)])
def test_fused_without_epilogue_is_bit_identical_to_plain(M, K, N):
    """NULL bias and no activation: the same kernels, the same bits."""
    A, Bq, S = make_inputs(M, K, N, 128, seed=M + 3)
    Bp = repack_on_device(dev(Bq), K, N)
    say("fused == plain", M, K, N, w4.w4a16_describe(M, K, N, 128))
    plain = run_gemm(A, Bq, S, 128, Bp=Bp)
    fused = run_gemm_fused(A, Bq, S, 128, None, w4.W4A16_ACT_NONE, Bp=Bp)
    assert np.array_equal(plain.view(np.uint16), fused.view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(2, 512, 64), (40, 1024, 208), (200, 512, 128)])
def test_fused_zero_activations_give_the_bias(M, K, N):
    """A = 0: every row is bias (no activation) or relu(bias), exactly, and
    SiLU(bias) within one FP16 ulp."""
    _, Bq, S = make_inputs(1, K, N, 128, seed=N)
    A = np.zeros((M, K), dtype=np.float16)
    bias = make_bias(N, seed=N + 1)
    Bp = repack_on_device(dev(Bq), K, N)
    say("fused zero rows", M, K, N, w4.w4a16_describe(M, K, N, 128))
    for name, act in ACTS.items():
        C = run_gemm_fused(A, Bq, S, 128, bias, act, Bp=Bp)
        want = oracle.activation(bias.astype(np.float64), act).astype(np.float16)
        if name == "silu":
            ulp = np.spacing(np.abs(want)).astype(np.float64)
            assert np.all(np.abs(C.astype(np.float64) - want.astype(np.float64)) <= ulp)
        else:
            assert np.array_equal(C, np.broadcast_to(want, C.shape)), name


def test_fused_full_size_sampled_columns():
    """The gate/up layer at its full size (M = 128, K = 4096, N = 22016), in
    the plan the step runs, SiLU with a bias, checked on sampled columns."""
    M, K, N = 128, 4096, 22016
    A, Bq, S = make_inputs(M, K, N, 128, seed=11)
    bias = make_bias(N, seed=12)
    say("fused full size", M, K, N, w4.w4a16_describe(M, K, N, 128))
    C = run_gemm_fused(A, Bq, S, 128, bias, w4.W4A16_ACT_SILU)
    cols = np.random.default_rng(13).choice(N, size=256, replace=False)
    cols = np.sort(np.concatenate([cols, [0, 15, 16, N - 1]]))
    C64 = oracle.gemm_columns(A, Bq, S, 128, cols)
    Z = C64 + bias[cols].astype(np.float64)[None, :]
    Y = oracle.activation(Z, oracle.ACT_SILU)
    assert_epilogue_close(C[:, cols], Z, Y, "gate/up sampled")


def test_fused_rejects_unknown_activation():
    import torch
    A = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    Bp = w4.alloc_packed(256, 64)
    S = torch.ones((2, 64), dtype=torch.float16, device="cuda")
    C = torch.empty((4, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm_fused(A, Bp, S, None, 7, C, 4, 256, 64, 128)
    assert e.value.name == "W4A16_ERR_EPILOGUE"
