"""Parity of the 8-bit weights (w8a16_repack, w8a16_dequant_debug,
w8a16_gemm) with the oracle.

Repack and dequantisation must match bit for bit; the GEMM must satisfy
``max|C - C_ref| <= 5e-3 max|C_ref| + ulp_fp16(max|C_ref|)`` against the
oracle's float64 sum through every kernel variant compiled for 8-bit codes,
and be exact where no rounding is left (one-hot rows, all codes 128).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs, make_words
from tests.gpu_util import dev, host_f16, host_u32, repack8_on_device, run_gemm8, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _words8(K, N, seed):
    """Uniform 8-bit codes: uniform uint32 words of [K/4][N] (two draws of
    the [K/8][N] word generator)."""
    return np.concatenate([make_words(K, N, seed), make_words(K, N, seed + 1)])


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (640, 48), (4096, 4096), (11008, 4096)])
def test_repack8_bit_exact(K, N):
    say("repack8", K, N)
    Bq8 = _words8(K, N, K + N)
    Bp = host_u32(repack8_on_device(dev(Bq8), K, N))
    assert np.array_equal(Bp, oracle.repack8(Bq8))


def _dequant8_gpu(Bq8, S, group):
    import torch
    K, N = Bq8.shape[0] * 4, Bq8.shape[1]
    Bp = repack8_on_device(dev(Bq8), K, N)
    W = torch.empty((K, N), dtype=torch.float16, device="cuda")
    w4.w8a16_dequant_debug(Bp, dev(S), W, K, N, group)
    torch.cuda.synchronize()
    return host_f16(W)


@pytest.mark.parametrize("K,N,group", [(128, 16, 128), (512, 80, 128), (1024, 64, 1024),
                                       (4096, 4096, 128)])
def test_dequant8_bit_exact(K, N, group):
    _, _, S = make_inputs(1, K, N, group, seed=K)
    Bq8 = _words8(K, N, K)
    say("dequant8", K, N, group)
    assert np.array_equal(_dequant8_gpu(Bq8, S, group).view(np.uint16),
                          oracle.dequant8(Bq8, S, group).view(np.uint16))


def test_dequant8_all_codes_against_every_scale():
    """All 256 codes against every finite nonzero FP16 scale of both signs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    scales = vals[np.isfinite(vals) & (vals != 0)]
    scales = np.concatenate([scales, np.ones((-scales.size) % 16, np.float16)])
    K = 256
    q = np.arange(256)[:, None] * np.ones((1, scales.size), dtype=np.int64)
    Bq8 = oracle.pack_codes8(q)
    S = scales[None, :]
    say("dequant8 exhaustive", scales.size)
    assert np.array_equal(_dequant8_gpu(Bq8, S, K).view(np.uint16),
                          oracle.dequant8(Bq8, S, K).view(np.uint16))


# the plans' kernels (as w8a16_describe prints them), one shape each
W8_CASES = [
    (1, 4096, 4096, "gemm_kernel<1,1,8,2>"),
    (1, 4096, 12288, "gemm_kernel<1,1,4,2>"),
    (1, 4096, 22016, "gemm_kernel<1,2,8,2>"),
    (1, 2048, 36864, "gemm_kernel<1,4,4,2>"),
    (8, 1024, 1024, "gemm_kernel<1,1,4,2>"),
    (8, 11008, 1024, "gemm_kernel<1,4,4,4>"),
    (8, 13824, 512, "gemm_kernel<1,4,4,2>"),
    (16, 1024, 8192, "gemm_lds_kernel<1,2,1,8,4>"),
    (32, 1024, 4096, "gemm_lds_kernel<2,2,1,8,4>"),
    (45, 1024, 208, "gemm_lds_kernel<4,1,1,8,3>"),
    (128, 1024, 1024, "gemm_lds_kernel<4,1,1,8,3>"),
    (128, 512, 36864, "gemm_lds_kernel<4,2,2,4,3>"),
    (128, 256, 65536, "gemm_lds_kernel<8,2,1,8,3>"),
    (300, 512, 512, "gemm_lds_kernel<8,2,1,8,3>"),
]


@pytest.mark.parametrize("M,K,N,kernel", W8_CASES)
def test_gemm8_matches_oracle(M, K, N, kernel):
    desc = w4.w8a16_describe(M, K, N, 128)
    assert desc.startswith(kernel + " "), desc
    A, _, S = make_inputs(M, K, N, 128, seed=M + N)
    Bq8 = _words8(K, N, M * 7 + N)
    say("gemm8", M, K, N, desc)
    C = run_gemm8(A, Bq8, S, 128)
    cols = None
    if N > 16384:
        cols = np.sort(np.concatenate([np.random.default_rng(N).choice(N, 192, replace=False),
                                       [0, 15, 16, N - 1]]))
    _, C64 = oracle.gemm8(A, Bq8, S, 128, cols=cols)
    assert_gemm_close(C if cols is None else C[:, cols], C64, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("plan", ["1,4,4,5,4", "1,2,8,3,2", "1,2,8,4,4,2", "2,2,8,2,4,2",
                                  "4,1,8,3,3,2", "4,2,4,2,3,2,0,2", "8,2,8,2,3,2"])
def test_gemm8_forced_plans_split_k(monkeypatch, plan):
    M, K, N, group = 45, 3584, 208, 512
    A, _, S = make_inputs(M, K, N, group, seed=5)
    Bq8 = _words8(K, N, 9)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w8a16_describe(M, K, N, group)
    assert "splits=1 " not in desc, desc
    say("gemm8 forced", plan, desc)
    C = run_gemm8(A, Bq8, S, group)
    _, C64 = oracle.gemm8(A, Bq8, S, group)
    assert_gemm_close(C, C64, f"plan {plan}")


@pytest.mark.parametrize("M,K,N", [(5, 384, 48), (70, 512, 64), (130, 256, 32)])
def test_gemm8_one_hot_rows_exact(M, K, N):
    _, _, S = make_inputs(1, K, N, 128, seed=M)
    Bq8 = _words8(K, N, M + 1)
    rng = np.random.default_rng(M + 2)
    ks = rng.integers(0, K, size=M)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), ks] = (2.0 ** rng.integers(-2, 3, size=M)).astype(np.float16)
    say("gemm8 one-hot", M, K, N)
    C = run_gemm8(A, Bq8, S, 128)
    C16, _ = oracle.gemm8(A, Bq8, S, 128)
    assert np.array_equal(C.astype(np.float64), C16.astype(np.float64))


def test_gemm8_all_codes_128_give_zero():
    A, _, S = make_inputs(17, 2048, 128, 128, seed=3)
    Bq8 = np.full((2048 // 4, 128), 0x80808080, dtype=np.uint32)
    say("gemm8 codes 128")
    assert not np.any(run_gemm8(A, Bq8, S, 128).astype(np.float64))


def test_gemm8_deterministic_split_k():
    import torch
    M, K, N = 16, 4096, 12288
    A, _, S = make_inputs(M, K, N, 128, seed=8)
    Bq8 = _words8(K, N, 10)
    desc = w4.w8a16_describe(M, K, N, 128)
    assert "splits=1 " not in desc, desc
    Bp = repack8_on_device(dev(Bq8), K, N)
    ws = w4.alloc_workspace8(M, K, N, 128)
    say("gemm8 determinism", desc)
    first = run_gemm8(A, Bq8, S, 128, workspace=ws, Bp=Bp)
    for i in range(8):
        again = run_gemm8(A, Bq8, S, 128, workspace=ws, Bp=Bp)
        assert np.array_equal(first.view(np.uint16), again.view(np.uint16)), f"run {i}"
    _, C64 = oracle.gemm8(A, Bq8, S, 128)
    assert_gemm_close(first, C64)
