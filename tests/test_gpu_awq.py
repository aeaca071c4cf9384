"""Parity of the zero-point and BF16 formats (w4a16_gemm_awq,
w4a16_dequant_awq_debug) with the oracle.

Dequantisation must match the oracle bit for bit.  The GEMM must satisfy
``max|C - C_ref| <= 5e-3 max|C_ref| + one ulp`` of the output type against
the oracle's float64 sum, through every kernel variant compiled for these
formats; FP16 without zero points must equal w4a16_gemm bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs_awq
from tests.gpu_util import dev, host_u16, repack_on_device, run_gemm, run_gemm_awq, say
from tests.tolerance import bf16_bound, gemm_bound

pytestmark = pytest.mark.gpu

# (format name, dtype, with zero points)
FORMATS = [("f16+zp", 0, True), ("bf16", 1, False), ("bf16+zp", 1, True)]


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _inputs(M, K, N, group, seed, dtype, zp):
    A, Bq, S, Z = make_inputs_awq(M, K, N, group, seed=seed, bf16=dtype == 1)
    return A, Bq, S, (Z if zp else None)


def _values(C, dtype):
    return oracle.bf16_to_f64(C) if dtype else np.asarray(C, dtype=np.float64)


def _check(C, C64, dtype, what):
    got = _values(C, dtype)
    assert np.all(np.isfinite(got)), what
    err = float(np.max(np.abs(got - C64))) if C64.size else 0.0
    bound = bf16_bound(C64) if dtype else gemm_bound(C64)
    assert err <= bound, f"{what}: max|C - C_ref| = {err:.4g} > {bound:.4g}"


def _dequant_gpu(Bq, S, Z, group, dtype):
    import torch
    K, N = Bq.shape[0] * 8, Bq.shape[1]
    Bp = repack_on_device(dev(Bq), K, N)
    W = torch.empty((K, N), dtype=torch.int16, device="cuda")
    Z_d = None if Z is None else torch.from_numpy(np.ascontiguousarray(Z)).cuda()
    w4.w4a16_dequant_awq_debug(Bp, dev(S), Z_d, W, K, N, group, dtype)
    torch.cuda.synchronize()
    return host_u16(W)


def _same(got_bits, want, dtype):
    return np.array_equal(got_bits, want.view(np.uint16))


@pytest.mark.parametrize("fmt,dtype,zp", FORMATS)
@pytest.mark.parametrize("K,N,group", [(128, 16, 128), (512, 80, 128), (1024, 64, 1024),
                                       (4096, 4096, 128)])
def test_awq_dequant_bit_exact(fmt, dtype, zp, K, N, group):
    _, Bq, S, Z = _inputs(1, K, N, group, K + N, dtype, zp)
    say("awq dequant", fmt, K, N, group)
    got = _dequant_gpu(Bq, S, Z, group, dtype)
    assert _same(got, oracle.dequant_awq(Bq, S, Z, group, dtype), dtype)


@pytest.mark.parametrize("fmt,dtype,zp", FORMATS)
def test_awq_dequant_exhaustive_codes_zero_points_scales(fmt, dtype, zp):
    """Every code against every zero point (16 x 16) for 2048 scales of both
    signs across the whole range, plus the extremes."""
    rng = np.random.default_rng(21)
    if dtype:
        sc = rng.integers(0, 2**16, size=4096, dtype=np.uint16)
        sc = sc[(((sc >> 7) & 0xFF) != 0xFF) & ((sc & 0x7FFF) != 0)][:2040]
        sc = np.concatenate([sc, np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x0080, 0xFF7F,
                                           0x3C00, 0x4000], np.uint16)])
    else:
        sc = rng.integers(0, 2**16, size=4096, dtype=np.uint16).view(np.float16)
        sc = sc[np.isfinite(sc) & (sc != 0)][:2040]
        sc = np.concatenate([sc, np.array([1.0, -1.0, 2**-24, 65504.0, -65504.0, 6.1e-5,
                                           0.0123, 3.0], np.float16)])
    ns = sc.size
    K = 128
    q = np.tile(np.arange(16), 8)[:, None] * np.ones((1, 16 * ns), dtype=np.int64)
    Bq = oracle.pack_codes(q)
    S = np.repeat(sc, 16)[None, :]
    Z = np.tile(np.arange(16, dtype=np.uint8), ns)[None, :] if zp else None
    say("awq dequant exhaustive", fmt, ns)
    got = _dequant_gpu(Bq, S, Z, K, dtype)
    assert _same(got, oracle.dequant_awq(Bq, S, Z, K, dtype), dtype)


# (M, K, N, the plan's kernel and template arguments as w4a16_describe prints them)
AWQ_CASES = [
    (1, 4096, 4096, "gemm_kernel<1,1,8,2>"),
    (1, 4096, 12288, "gemm_kernel<1,1,8,2>"),
    (1, 4096, 22016, "gemm_kernel<1,2,8,2>"),
    (1, 2048, 36864, "gemm_kernel<1,4,4,2>"),
    (8, 1024, 1024, "gemm_kernel<1,2,8,2>"),
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
SAMPLE_COLS_ABOVE = 16384   # wider layers are checked on sampled columns


@pytest.mark.parametrize("fmt,dtype,zp", FORMATS)
@pytest.mark.parametrize("M,K,N,kernel", AWQ_CASES)
def test_awq_gemm_matches_oracle(fmt, dtype, zp, M, K, N, kernel):
    desc = w4.w4a16_describe(M, K, N, 128)
    assert desc.startswith(kernel + " "), desc   # each compiled variant is exercised
    A, Bq, S, Z = _inputs(M, K, N, 128, M * 3 + N, dtype, zp)
    say("awq gemm", fmt, M, K, N, desc)
    C = run_gemm_awq(A, Bq, S, Z, 128, dtype)
    cols = None
    if N > SAMPLE_COLS_ABOVE:
        cols = np.sort(np.concatenate([np.random.default_rng(N).choice(N, 192, replace=False),
                                       [0, 15, 16, N - 1]]))
    _, C64 = oracle.gemm_awq(A, Bq, S, Z, 128, dtype, cols=cols)
    _check(C if cols is None else C[:, cols], C64, dtype, f"{fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt,dtype,zp", FORMATS)
@pytest.mark.parametrize("plan", ["1,4,4,5,4", "1,2,8,3,2", "1,1,8,2,2", "1,2,8,4,4,2",
                                  "2,2,8,2,4,2", "4,1,8,3,3,2", "4,2,4,2,3,2,0,2",
                                  "8,2,8,2,3,2", "1,4,8,5,4,4", "2,4,8,4,3,4", "4,4,8,3,3,4"])
def test_awq_forced_plans_split_k(monkeypatch, fmt, dtype, zp, plan):
    """The compiled variants with split-K (forced; for the stream-K kernel,
    grids that share tiles between workgroups), M = 45 ragged rows, N = 208
    a ragged column tile, group 512."""
    M, K, N, group = 45, 3584, 208, 512
    A, Bq, S, Z = _inputs(M, K, N, group, 5, dtype, zp)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, group)
    assert "splits=1 " not in desc, desc
    say("awq forced", fmt, plan, desc)
    C = run_gemm_awq(A, Bq, S, Z, group, dtype)
    _, C64 = oracle.gemm_awq(A, Bq, S, Z, group, dtype)
    _check(C, C64, dtype, f"{fmt} plan {plan}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (16, 4096, 12288), (45, 3584, 208),
                                   (128, 4096, 4096), (300, 1024, 512)])
def test_awq_f16_without_zero_points_is_the_plain_gemm(M, K, N):
    A, Bq, S, _ = make_inputs_awq(M, K, N, 128, seed=M + 1)
    Bp = repack_on_device(dev(Bq), K, N)
    say("awq f16 == plain", M, K, N)
    plain = run_gemm(A, Bq, S, 128, Bp=Bp)
    awq = run_gemm_awq(A, Bq, S, None, 128, 0, Bp=Bp)
    assert np.array_equal(plain.view(np.uint16), awq.view(np.uint16))


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("M,K,N", [(1, 2048, 1024), (45, 1024, 208), (128, 1024, 1024)])
def test_awq_zero_points_eight_equal_the_symmetric_format(dtype, M, K, N):
    A, Bq, S, Z = make_inputs_awq(M, K, N, 128, seed=N, bf16=dtype == 1)
    Z8 = np.full_like(Z, 8)
    Bp = repack_on_device(dev(Bq), K, N)
    say("awq z=8", dtype, M, K, N)
    a = run_gemm_awq(A, Bq, S, None, 128, dtype, Bp=Bp)
    b = run_gemm_awq(A, Bq, S, Z8, 128, dtype, Bp=Bp)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("dtype", [0, 1])
def test_awq_codes_at_their_zero_points_give_zero(dtype):
    A, _, S, Z = make_inputs_awq(45, 1024, 208, 128, seed=2, bf16=dtype == 1)
    Bq = oracle.pack_codes(np.repeat(Z, 128, axis=0))
    say("awq q == z", dtype)
    C = run_gemm_awq(A, Bq, S, Z, 128, dtype)
    assert not np.any(_values(C, dtype))


def test_awq_split_k_deterministic():
    import torch
    M, K, N = 16, 4096, 12288
    A, Bq, S, Z = make_inputs_awq(M, K, N, 128, seed=7, bf16=True)
    desc = w4.w4a16_describe(M, K, N, 128)
    assert "splits=1 " not in desc, desc
    Bp = repack_on_device(dev(Bq), K, N)
    ws = w4.alloc_workspace(M, K, N, 128)
    say("awq determinism", desc)
    first = run_gemm_awq(A, Bq, S, Z, 128, 1, workspace=ws, Bp=Bp)
    for i in range(8):
        again = run_gemm_awq(A, Bq, S, Z, 128, 1, workspace=ws, Bp=Bp)
        assert np.array_equal(first, again), f"run {i}"


def test_awq_forced_plan_outside_the_compiled_variants_is_ignored(monkeypatch):
    """A forced plan naming a variant compiled for no dense format (here a
    2:4-only LDS tile) leaves the heuristic's plan in place, for FP16 and
    BF16 alike, and the call runs it."""
    M, K, N = 45, 1024, 208
    heur = w4.w4a16_describe(M, K, N, 128)
    w4.w4a16_set_forced_plan("4,2,4,1,3,2")
    assert w4.w4a16_describe(M, K, N, 128) == heur
    say("awq ignored plan", heur)
    for dtype in (1, 0):
        A, Bq, S, Z = make_inputs_awq(M, K, N, 128, seed=3, bf16=bool(dtype))
        C = run_gemm_awq(A, Bq, S, Z, 128, dtype)
        _, C64 = oracle.gemm_awq(A, Bq, S, Z, 128, dtype)
        _check(C, C64, dtype, f"dtype {dtype} ignored plan")