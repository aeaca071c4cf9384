"""The plan heuristic on the CPU (w4a16_plan_describe takes the compute-unit
count as an argument, so no device is needed): which kernel each batch and
layer size gets."""

from __future__ import annotations

import pytest

import weight_only_int4_gemm_amd as w4

CUS = 256  # MI355X

F16, F16ZP, BF16, BF16ZP, W8, SP24 = range(6)


def plan(M, K, N, fmt=F16, group=128):
    return w4.w4a16_plan_describe(M, K, N, group, fmt, CUS)


def test_stream_k_takes_9_to_64_rows_on_large_layers():
    K, N = 18432, 73728
    for M, name in ((9, "1,4,4,1,8"), (16, "1,4,4,1,8"), (17, "2,4,3,1,8"), (32, "2,4,3,1,8"),
                    (33, "4,4,3,1,8"), (64, "4,4,3,1,8")):
        for fmt in (F16, F16ZP, BF16, BF16ZP):
            assert plan(M, K, N, fmt).startswith(f"gemm_sk_kernel<{name}>"), (M, fmt)
        assert not plan(M, K, N, W8).startswith("gemm_sk_kernel<"), M
        assert not plan(M, K, N, SP24).startswith("gemm_sk_kernel<"), M
    for M in (1, 8, 65, 128, 1024):
        assert not plan(M, K, N).startswith("gemm_sk_kernel<"), M
    for K2, N2 in ((4096, 4096), (4096, 12288), (4096, 22016), (11008, 4096), (8192, 28672),
                   (28672, 8192), (13824, 5120)):
        for M in (16, 32, 64):
            assert not plan(M, K2, N2).startswith("gemm_sk_kernel<"), (M, K2, N2)


def test_plan_describe_checks_its_arguments():
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4096, 4096, 128, 6, CUS)    # no such format
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4096, 4096, 128, F16, 0)    # no compute units
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4000, 4096, 128, F16, CUS)  # K not a multiple of 128
