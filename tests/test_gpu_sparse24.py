"""Parity of the 2:4-sparse weights (w4a16_sparse24_repack,
w4a16_sparse24_dequant_debug, w4a16_sparse24_gemm) with the oracle.

Repack and dequantisation must match bit for bit (positive scales; with
negative scales a free slot's zero may carry the scale's sign, so zeros are
compared numerically there); the GEMM must satisfy ``max|C - C_ref| <=
5e-3 max|C_ref| + ulp_fp16(max|C_ref|)`` against the oracle's float64 sum
through every kernel variant compiled for the sparse format, and be exact
where no rounding is left (one-hot rows, empty masks).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs, make_mask24
from tests.gpu_util import dev, host_f16, host_u32, repack_sp24_on_device, run_gemm_sp24, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


@pytest.mark.parametrize("K,N,exact", [(128, 16, True), (256, 64, False), (640, 48, True),
                                       (4096, 4096, True), (11008, 4096, False)])
def test_repack_sp24_bit_exact(K, N, exact):
    _, Bq, _ = make_inputs(1, K, N, 128, seed=K + N)
    mask = make_mask24(K, N, seed=K, exact=exact)
    say("repack sp24", K, N, exact)
    Bp = host_u32(repack_sp24_on_device(dev(Bq), dev(mask), K, N))
    assert np.array_equal(Bp, oracle.repack_sparse24(Bq, mask))


def _dequant_gpu(Bq, mask, S, group):
    import torch
    K, N = Bq.shape[0] * 8, Bq.shape[1]
    Bp = repack_sp24_on_device(dev(Bq), dev(mask), K, N)
    W = torch.full((K, N), float("nan"), dtype=torch.float16, device="cuda")
    w4.w4a16_sparse24_dequant_debug(Bp, dev(S), W, K, N, group)
    torch.cuda.synchronize()
    return host_f16(W)


@pytest.mark.parametrize("K,N,group,exact", [(128, 16, 128, True), (512, 80, 128, False),
                                             (1024, 64, 1024, True), (4096, 4096, 128, True)])
def test_dequant_sp24_bit_exact(K, N, group, exact):
    _, Bq, S = make_inputs(1, K, N, group, seed=K)
    mask = make_mask24(K, N, seed=K + 1, exact=exact)
    say("dequant sp24", K, N, group, exact)
    assert np.array_equal(_dequant_gpu(Bq, mask, S, group).view(np.uint16),
                          oracle.dequant_sparse24(Bq, mask, S, group).view(np.uint16))


def test_dequant_sp24_every_code_position_and_scale_sign():
    """Every code at every slot position, masks of every byte value, FP16
    scales of both signs across the exponent range: nonzero weights bit for
    bit, zeros as numbers (a free slot's zero takes the scale's sign)."""
    K, N = 1024, 512
    rng = np.random.default_rng(7)
    Bq = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    mask = np.arange(K // 4 * N, dtype=np.int64).reshape(K // 4, N).astype(np.uint8)
    mag = (2.0 ** rng.uniform(-24, 15.9, size=(K // 128, N))).astype(np.float16)
    S = (mag * np.where(rng.integers(0, 2, size=mag.shape) == 1, -1, 1)).astype(np.float16)
    S[S == 0] = np.float16(1.0)
    say("dequant sp24 signs")
    W = _dequant_gpu(Bq, mask, S, 128)
    ref = oracle.dequant_sparse24(Bq, mask, S, 128)
    nz = ref != 0
    assert np.array_equal(W[nz].view(np.uint16), ref[nz].view(np.uint16))
    assert np.all(W[~nz] == 0)


def test_dequant_sp24_keeps_exactly_the_mask():
    K, N = 512, 64
    A, Bq, S = make_inputs(1, K, N, 128, seed=3)
    mask = make_mask24(K, N, seed=4)
    # codes 0 (weight -8 s, never zero) everywhere: the nonzeros are the mask
    Bq0 = np.zeros_like(Bq)
    say("dequant sp24 support")
    W = _dequant_gpu(Bq0, mask, S, 128)
    assert np.array_equal(W != 0, oracle.sparse24_keep(mask))


# the plans' kernels (as w4a16_sparse24_describe prints them), one shape each
SP_CASES = [
    (1, 4096, 4096, "gemm_kernel<1,1,8,2>"),
    (1, 4096, 12288, "gemm_kernel<1,1,4,2>"),
    (1, 4096, 22016, "gemm_kernel<1,2,8,2>"),
    (1, 2048, 36864, "gemm_kernel<1,4,4,2>"),
    (3, 13824, 4096, "gemm_kernel<1,2,8,2>"),
    (8, 1024, 1024, "gemm_kernel<1,1,4,2>"),
    (8, 11008, 1024, "gemm_kernel<1,4,4,2>"),
    (8, 13824, 512, "gemm_kernel<1,4,4,2>"),
    (16, 1024, 8192, "gemm_lds_kernel<1,2,1,8,4>"),
    (32, 1024, 4096, "gemm_lds_kernel<2,2,1,8,4>"),
    (45, 1024, 208, "gemm_lds_kernel<4,2,1,4,3>"),
    (128, 1024, 1024, "gemm_lds_kernel<4,2,1,4,3>"),
    (128, 512, 36864, "gemm_lds_kernel<4,2,1,4,3>"),
    (128, 256, 65536, "gemm_lds_kernel<4,2,1,4,3>"),
    (300, 512, 512, "gemm_lds_kernel<8,2,1,8,3>"),
]


@pytest.mark.parametrize("M,K,N,kernel", SP_CASES)
def test_gemm_sp24_matches_oracle(M, K, N, kernel):
    desc = w4.w4a16_sparse24_describe(M, K, N, 128)
    assert desc.startswith(kernel + " "), desc
    A, Bq, S = make_inputs(M, K, N, 128, seed=M + N)
    mask = make_mask24(K, N, seed=M * 7 + N)
    say("gemm sp24", M, K, N, desc)
    C = run_gemm_sp24(A, Bq, mask, S, 128)
    cols = None
    if N > 16384:
        cols = np.sort(np.concatenate([np.random.default_rng(N).choice(N, 192, replace=False),
                                       [0, 15, 16, N - 1]]))
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, 128, cols=cols)
    assert_gemm_close(C if cols is None else C[:, cols], C64, f"M={M} K={K} N={N}")


# every 2:4 variant the library compiles, each with a K split
@pytest.mark.parametrize("plan", ["1,1,8,3,2", "1,2,8,4,2", "1,1,4,5,2", "1,4,4,2,2",
                                  "1,2,8,4,4,2", "2,2,8,2,4,2", "8,2,8,2,3,2", "4,2,4,2,3,2",
                                  "4,2,4,3,3,2"])
def test_gemm_sp24_forced_plans_split_k(monkeypatch, plan):
    M, K, N, group = 45, 3584, 208, 512
    A, Bq, S = make_inputs(M, K, N, group, seed=5)
    mask = make_mask24(K, N, seed=6, exact=False)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_sparse24_describe(M, K, N, group)
    f = [int(x) for x in plan.split(",")] + [0, 0, 0]
    mb, nb, wk, depth, tile, wm = f[0], f[1], f[2], f[4], f[5], f[7] or 1
    want = (f"gemm_lds_kernel<{mb},{nb},{wm},{wk},{depth}>" if tile == 2
            else f"gemm_kernel<{mb},{nb},{wk},{depth}>")
    assert desc.startswith(want), desc
    assert "splits=1 " not in desc, desc
    say("gemm sp24 forced", plan, desc)
    C = run_gemm_sp24(A, Bq, mask, S, group)
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, group)
    assert_gemm_close(C, C64, f"plan {plan}")


@pytest.mark.parametrize("M,K,N", [(5, 384, 48), (70, 512, 64), (130, 256, 32)])
def test_gemm_sp24_one_hot_rows_exact(M, K, N):
    _, Bq, S = make_inputs(1, K, N, 128, seed=M)
    mask = make_mask24(K, N, seed=M + 3, exact=False)
    rng = np.random.default_rng(M + 2)
    ks = rng.integers(0, K, size=M)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), ks] = (2.0 ** rng.integers(-2, 3, size=M)).astype(np.float16)
    say("gemm sp24 one-hot", M, K, N)
    C = run_gemm_sp24(A, Bq, mask, S, 128)
    C16, _ = oracle.gemm_sparse24(A, Bq, mask, S, 128)
    assert np.array_equal(C.astype(np.float64), C16.astype(np.float64))


def test_gemm_sp24_empty_mask_gives_zero_and_full_mask_keeps_two():
    M, K, N = 17, 2048, 128
    A, Bq, S = make_inputs(M, K, N, 128, seed=3)
    say("gemm sp24 empty / full masks")
    zero = np.zeros((K // 4, N), dtype=np.uint8)
    assert not np.any(run_gemm_sp24(A, Bq, zero, S, 128).astype(np.float64))
    full = np.full((K // 4, N), 0xFF, dtype=np.uint8)
    low2 = np.full((K // 4, N), 0b0011, dtype=np.uint8)
    assert np.array_equal(run_gemm_sp24(A, Bq, full, S, 128).view(np.uint16),
                          run_gemm_sp24(A, Bq, low2, S, 128).view(np.uint16))


def test_gemm_sp24_group_k_equals_replicated_groups():
    M, K, N = 9, 1024, 64
    A, Bq, S = make_inputs(M, K, N, K, seed=12)
    mask = make_mask24(K, N, seed=13)
    say("gemm sp24 group = K")
    C_k = run_gemm_sp24(A, Bq, mask, S, K)
    C_128 = run_gemm_sp24(A, Bq, mask, np.repeat(S, K // 128, axis=0), 128)
    assert np.array_equal(C_k.view(np.uint16), C_128.view(np.uint16))
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, K)
    assert_gemm_close(C_k, C64)


def test_gemm_sp24_deterministic_split_k():
    M, K, N = 16, 11008, 4096
    A, Bq, S = make_inputs(M, K, N, 128, seed=8)
    mask = make_mask24(K, N, seed=10)
    desc = w4.w4a16_sparse24_describe(M, K, N, 128)
    assert "splits=1 " not in desc, desc
    Bp = repack_sp24_on_device(dev(Bq), dev(mask), K, N)
    ws = w4.alloc_workspace_sparse24(M, K, N, 128)
    say("gemm sp24 determinism", desc)
    first = run_gemm_sp24(A, Bq, mask, S, 128, workspace=ws, Bp=Bp)
    for i in range(8):
        again = run_gemm_sp24(A, Bq, mask, S, 128, workspace=ws, Bp=Bp)
        assert np.array_equal(first.view(np.uint16), again.view(np.uint16)), f"run {i}"
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, 128)
    assert_gemm_close(first, C64)


# Llama-2-7B layer shapes at the workload's batch sizes, on sampled columns
@pytest.mark.parametrize("K,N", [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)])
@pytest.mark.parametrize("M", [1, 16, 128])
def test_gemm_sp24_llama_shapes_sampled(M, K, N):
    A, Bq, S = make_inputs(M, K, N, 128, seed=0)
    mask = make_mask24(K, N, seed=1)
    desc = w4.w4a16_sparse24_describe(M, K, N, 128)
    say("gemm sp24 llama", M, K, N, desc)
    C = run_gemm_sp24(A, Bq, mask, S, 128)
    cols = np.sort(np.concatenate([np.random.default_rng(M + N).choice(N, 256, replace=False),
                                   [0, 15, 16, N - 1]]))
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, 128, cols=cols)
    assert_gemm_close(C[:, cols], C64, f"M={M} K={K} N={N}")


# The workload's other shapes at full size, in the plans the benchmark times:
# every row, a sample of output columns (first, middle and last column tiles
# and random ones), each computed by the oracle.
def _sample_cols(N, count, seed):
    rng = np.random.default_rng(seed)
    cols = set(range(0, 16)) | set(range(N - 16, N)) | set(range(N // 2, N // 2 + 16))
    cols |= set(rng.choice(N, size=count, replace=False).tolist())
    return np.array(sorted(cols))


def _sampled_sp24(K, N, group, Ms, seed, count=64):
    import torch
    _, Bq, S = make_inputs(1, K, N, group, seed=seed)
    mask = make_mask24(K, N, seed=seed + 1)
    Bp = repack_sp24_on_device(dev(Bq), dev(mask), K, N)
    cols = _sample_cols(N, count, seed)
    for M in Ms:
        A, _, _ = make_inputs(M, K, 8, group, seed=seed + M)
        say("sp24 sampled", K, N, group, "M", M, w4.w4a16_sparse24_describe(M, K, N, group))
        C = run_gemm_sp24(A, Bq, mask, S, group, Bp=Bp)
        _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, group, cols=cols)
        assert_gemm_close(C[:, cols], C64, f"K={K} N={N} g={group} M={M}")
    del Bp
    torch.cuda.empty_cache()


def test_gemm_sp24_large_layer_batch_sweep():
    _sampled_sp24(18432, 73728, 128, (1, 2, 4, 8, 16, 32, 64, 128), seed=0)


def test_gemm_sp24_prefill_layer():
    _sampled_sp24(8192, 28672, 128, (512, 1024, 4096), seed=0, count=32)


@pytest.mark.parametrize("K,N", [(28672, 8192), (13824, 5120)])
@pytest.mark.parametrize("per_channel", [False, True])
def test_gemm_sp24_deep_k_layers(K, N, per_channel):
    _sampled_sp24(K, N, K if per_channel else 128, (1, 8, 32), seed=0)
