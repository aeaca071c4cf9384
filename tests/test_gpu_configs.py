"""Parity at the full workload sizes, in the launch configuration the
benchmark times (the library's own plan).

Small layers are compared element by element against the whole oracle
product; for the largest matrices the oracle computes a sample of output
columns (every row) one column at a time, spread over the first, last and
interior column tiles.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs
from tests.gpu_util import dev, repack_on_device, run_gemm, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu

# Llama-2-7B-shaped layers (K x N): fused qkv, o, fused gate/up, down.
LLAMA_LAYERS = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _sample_cols(N, count, seed):
    rng = np.random.default_rng(seed)
    cols = set(range(0, 16)) | set(range(N - 16, N)) | set(range(N // 2, N // 2 + 16))
    cols |= set(rng.choice(N, size=count, replace=False).tolist())
    return np.array(sorted(cols))


def test_single_layer_4096_m16():
    M, K, N = 16, 4096, 4096
    A, Bq, S = make_inputs(M, K, N, 128, seed=0)
    say("4096x4096 M=16")
    C = run_gemm(A, Bq, S, 128)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    assert_gemm_close(C, C64, "4096x4096 M=16")


@pytest.mark.parametrize("K,N", LLAMA_LAYERS)
def test_llama_layers(K, N):
    import torch
    _, Bq, S = make_inputs(1, K, N, 128, seed=0)
    Bp = repack_on_device(dev(Bq), K, N)
    for M in (1, 16, 128):
        A, _, _ = make_inputs(M, K, 8, 128, seed=M)
        say("llama layer", K, N, "M", M)
        C = run_gemm(A, Bq, S, 128, Bp=Bp)
        _, C64 = oracle.gemm(A, Bq, S, 128)
        assert_gemm_close(C, C64, f"K={K} N={N} M={M}")
    del Bp
    torch.cuda.empty_cache()


def _sampled(K, N, group, Ms, seed, count=96):
    import torch
    _, Bq, S = make_inputs(1, K, N, group, seed=seed)
    Bp = repack_on_device(dev(Bq), K, N)
    cols = _sample_cols(N, count, seed)
    for M in Ms:
        A, _, _ = make_inputs(M, K, 8, group, seed=seed + M)
        say("sampled", K, N, group, "M", M)
        C = run_gemm(A, Bq, S, group, Bp=Bp)
        ref = oracle.gemm_columns(A, Bq, S, group, cols)
        assert_gemm_close(C[:, cols], ref, f"K={K} N={N} g={group} M={M}")
    del Bp
    torch.cuda.empty_cache()


def test_large_layer_batch_sweep():
    _sampled(18432, 73728, 128, (1, 2, 4, 8, 16, 32, 64, 128), seed=0)


def test_prefill_layer():
    _sampled(8192, 28672, 128, (512, 1024, 4096), seed=0, count=48)


@pytest.mark.parametrize("K,N", [(28672, 8192), (13824, 5120)])
@pytest.mark.parametrize("per_channel", [False, True])
def test_deep_k_layers(K, N, per_channel):
    _sampled(K, N, K if per_channel else 128, (1, 8, 32), seed=0)
