"""The stream-K kernel (gemm_sk.hpp) against the oracle: every compiled
variant, grids that cut tiles between workgroups anywhere (so partial tiles
go through the workspace and the last arriver adds them in K order), tile
padding when the K blocks are not a multiple of the pipeline depth, ragged
rows and columns, determinism, workspace reuse and the fused output stage."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_bias, make_inputs
from tests.gpu_util import dev, repack_on_device, run_gemm, run_gemm_fused, say
from tests.tolerance import assert_epilogue_close, assert_gemm_close

pytestmark = pytest.mark.gpu

# compiled variants: 16*mb rows, 16*nb columns per wave, pipeline depth ns,
# eight waves
VARIANTS = [(1, 4, 4), (2, 4, 3), (4, 4, 3), (8, 2, 3)]


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _plan(mb, ns, grid, nb=4):
    return f"{mb},{nb},8,{grid},{ns},4"


def _name(mb, ns, nb=4):
    return f"gemm_sk_kernel<{mb},{nb},{ns},8>"


@pytest.mark.parametrize("mb,nb,ns", VARIANTS)
@pytest.mark.parametrize("grid", [1, 3, 7, 0])
def test_sk_forced_grids_agree(mb, nb, ns, grid):
    """M = 45 and N = 208 leave ragged row and column tiles; K = 3584 is 28
    K blocks (padded to a multiple of ns where needed); grids of 3 and 7
    workgroups cut tiles in the middle."""
    M, K, N, g = 45, 3584, 208, 128
    A, Bq, S = make_inputs(M, K, N, g, seed=11)
    w4.w4a16_set_forced_plan(_plan(mb, ns, grid, nb))
    desc = w4.w4a16_describe(M, K, N, g)
    assert desc.startswith(_name(mb, ns, nb)), desc
    say("sk forced", mb, nb, ns, grid, desc)
    C = run_gemm(A, Bq, S, g)
    _, C64 = oracle.gemm(A, Bq, S, g)
    assert_gemm_close(C, C64, desc)


@pytest.mark.parametrize("M,K,N,mb,nb,ns", [(16, 2048, 4160, 1, 4, 4), (40, 2048, 4160, 2, 4, 3),
                                            (64, 3840, 768, 4, 4, 3), (130, 1152, 2048, 4, 4, 3),
                                            (16, 1536, 1536, 1, 4, 4), (200, 4096, 1024, 8, 2, 3),
                                            (300, 1152, 2096, 8, 2, 3)])
def test_sk_default_and_split_grids(M, K, N, mb, nb, ns):
    """Several column and row tiles; the default grid (one workgroup per
    compute unit, at least eight K blocks each) and a 5-workgroup grid whose
    runs end inside tiles."""
    A, Bq, S = make_inputs(M, K, N, 128, seed=M + N)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    w4.w4a16_set_forced_plan(_plan(mb, ns, 0, nb))
    desc = w4.w4a16_describe(M, K, N, 128)
    assert desc.startswith(_name(mb, ns, nb)), desc
    say("sk default grid", M, K, N, desc)
    assert_gemm_close(run_gemm(A, Bq, S, 128), C64, desc)
    w4.w4a16_set_forced_plan(_plan(mb, ns, 5, nb))
    desc5 = w4.w4a16_describe(M, K, N, 128)
    assert "workspace=0" not in desc5, desc5
    say("sk grid 5", M, K, N, desc5)
    assert_gemm_close(run_gemm(A, Bq, S, 128), C64, desc5)


def test_sk_group_k_and_coarse_groups():
    """Per-column scales (group = K) and groups of four K blocks."""
    M, K, N = 72, 2560, 512
    for g in (K, 512):
        A, Bq, S = make_inputs(M, K, N, g, seed=g)
        w4.w4a16_set_forced_plan(_plan(4, 3, 3))
        desc = w4.w4a16_describe(M, K, N, g)
        say("sk group", g, desc)
        C = run_gemm(A, Bq, S, g)
        _, C64 = oracle.gemm(A, Bq, S, g)
        assert_gemm_close(C, C64, f"group {g} {desc}")


def test_sk_one_hot_rows_are_exact():
    """A row that is e_k picks weight row k exactly (every other product is an
    exact zero), through partial tiles and padding: the reduction adds exact
    zeros in any order."""
    M, K, N, g = 40, 1280, 320, 128
    _, Bq, S = make_inputs(M, K, N, g, seed=3)
    A = np.zeros((M, K), dtype=np.float16)
    ks = np.random.default_rng(4).integers(0, K, size=M)
    A[np.arange(M), ks] = 1.0
    W = oracle.dequant(Bq, S, g)
    for mb, nb, ns in VARIANTS:
        w4.w4a16_set_forced_plan(_plan(mb, ns, 4, nb))
        say("sk one-hot", mb, nb, ns)
        C = run_gemm(A, Bq, S, g)
        assert np.array_equal(C.astype(np.float64), W[ks].astype(np.float64)), (mb, nb, ns)


def test_sk_deterministic_and_counters_reset():
    """Repeats are bit-identical on a shared workspace, whose counter header
    is all zero after every call."""
    import torch
    M, K, N, g = 96, 4096, 2048, 128
    A, Bq, S = make_inputs(M, K, N, g, seed=5)
    w4.w4a16_set_forced_plan(_plan(4, 3, 7))
    desc = w4.w4a16_describe(M, K, N, g)
    need = w4.w4a16_workspace_bytes(M, K, N, g)
    assert need > 65536, desc
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Bp = repack_on_device(dev(Bq), K, N)
    say("sk determinism", desc)
    first = run_gemm(A, Bq, S, g, workspace=ws, Bp=Bp)
    for i in range(8):
        again = run_gemm(A, Bq, S, g, workspace=ws, Bp=Bp)
        assert np.array_equal(first.view(np.uint16), again.view(np.uint16)), i
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    _, C64 = oracle.gemm(A, Bq, S, g)
    assert_gemm_close(first, C64, desc)


@pytest.mark.parametrize("act", [0, 1, 2])
def test_sk_fused_epilogue(act):
    """Bias and ReLU / SiLU in the stream-K output stage, whole and shared
    tiles alike."""
    M, K, N, g = 45, 3584, 208, 128
    A, Bq, S = make_inputs(M, K, N, g, seed=9)
    bias = make_bias(N, seed=10)
    _, Y64, Z64 = oracle.gemm_fused(A, Bq, S, g, bias, act)
    for grid, (mb, nb, ns) in ((1, (2, 4, 3)), (5, (2, 4, 3)), (5, (1, 4, 4)), (7, (4, 4, 3)),
                               (3, (8, 2, 3))):
        w4.w4a16_set_forced_plan(_plan(mb, ns, grid, nb))
        desc = w4.w4a16_describe(M, K, N, g)
        say("sk fused", act, desc)
        C = run_gemm_fused(A, Bq, S, g, bias, act)
        assert_epilogue_close(C, Z64, Y64, f"act {act} {desc}")


def test_forced_plan_without_stream_k():
    """The forced plan "tile -1" gives the plan the heuristic makes without
    the stream-K kernel, and it runs."""
    w4.w4a16_set_forced_plan("0,0,0,0,0,-1")
    desc = w4.w4a16_describe(16, 18432, 73728, 128)
    assert not desc.startswith("gemm_sk_kernel<"), desc
    M = 64
    A, Bq, S = make_inputs(M, 2048, 4096, 128, seed=8)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    say("tile -1", w4.w4a16_describe(M, 2048, 4096, 128))
    assert_gemm_close(run_gemm(A, Bq, S, 128), C64, "tile -1")


@pytest.mark.parametrize("mb,nb,ns", VARIANTS)
@pytest.mark.parametrize("M,K,N", [(20, 128, 16), (100, 256, 48), (9, 384, 528), (128, 640, 1040)])
def test_sk_small_k_and_narrow_n(mb, nb, ns, M, K, N):
    """K blocks fewer than the pipeline stages (all but one iteration of a
    tile is padding), a single 16-column block, and N one block past a tile
    boundary, on the default and a 3-workgroup grid."""
    A, Bq, S = make_inputs(M, K, N, 128, seed=M + K + N)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    for grid in (0, 3):
        w4.w4a16_set_forced_plan(_plan(mb, ns, grid, nb))
        desc = w4.w4a16_describe(M, K, N, 128)
        assert desc.startswith(_name(mb, ns, nb)), desc
        say("sk small", M, K, N, desc)
        assert_gemm_close(run_gemm(A, Bq, S, 128), C64, desc)
