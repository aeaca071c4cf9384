"""Parity of the HIP path with the oracle, through the C interface.

Repack and dequantisation must match bit for bit.  The GEMM must satisfy
``max|C - C_ref| <= 5e-3 * max|C_ref| + ulp_fp16(max|C_ref|)`` against the
oracle's float64-accumulated product, and be exact where the arithmetic
leaves no rounding (one-hot activation rows, all codes 8).
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs
from tests.gpu_util import dev, host_f16, host_u32, repack_on_device, run_gemm, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


# ---------------------------------------------------------------------------
# repack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (640, 48), (4096, 4096),
                                 (11008, 4096), (4096, 22016)])
def test_repack_bit_exact(K, N):
    say("repack", K, N)
    Bq = np.random.default_rng(K * 7 + N).integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    Bp = host_u32(repack_on_device(dev(Bq), K, N))
    assert np.array_equal(Bp, oracle.repack(Bq))
    assert np.array_equal(oracle.unrepack(Bp, K, N), Bq)


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------

def _dequant_gpu(Bq, S, group):
    import torch
    K, N = Bq.shape[0] * 8, Bq.shape[1]
    Bp = repack_on_device(dev(Bq), K, N)
    W = torch.empty((K, N), dtype=torch.float16, device="cuda")
    w4.w4a16_dequant_debug(Bp, dev(S), W, K, N, group)
    torch.cuda.synchronize()
    return host_f16(W)


def _same_bits(x, y):
    return np.array_equal(x.view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("K,N,group", [(128, 16, 128), (512, 80, 128), (1024, 64, 1024),
                                       (4096, 4096, 128), (13824, 5120, 13824)])
def test_dequant_bit_exact(K, N, group):
    say("dequant", K, N, group)
    _, Bq, S = make_inputs(1, K, N, group, seed=K + N)
    assert _same_bits(_dequant_gpu(Bq, S, group), oracle.dequant(Bq, S, group))


def test_dequant_exhaustive_codes_and_scales():
    """All 16 codes against every finite nonzero FP16 scale, both signs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    scales = vals[np.isfinite(vals) & (vals != 0)]
    pad = (-scales.size) % 16
    scales = np.concatenate([scales, np.ones(pad, np.float16)])
    K = 128
    q = np.repeat(np.tile(np.arange(16), K // 16)[:, None], scales.size, axis=1)
    Bq = oracle.pack_codes(q)
    S = scales[None, :].astype(np.float16)
    say("dequant exhaustive", K, scales.size)
    got = _dequant_gpu(Bq, S, K)
    assert _same_bits(got, oracle.dequant(Bq, S, K))


def test_repack_then_unit_scale_gives_centred_codes():
    K, N = 1024, 256
    _, Bq, _ = make_inputs(1, K, N, 128, seed=99)
    S = np.ones((K // 128, N), dtype=np.float16)
    say("unit scale", K, N)
    W = _dequant_gpu(Bq, S, 128)
    assert np.array_equal(W.astype(np.int64), oracle.unpack_codes(Bq).astype(np.int64) - 8)


# ---------------------------------------------------------------------------
# GEMM: exact cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(5, 384, 48), (20, 1024, 256), (70, 512, 64), (130, 256, 32)])
def test_gemm_one_hot_rows_exact(M, K, N):
    _, Bq, S = make_inputs(1, K, N, 128, seed=M)
    rng = np.random.default_rng(M + 1)
    ks = rng.integers(0, K, size=M)
    ps = rng.integers(-2, 3, size=M)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), ks] = (2.0 ** ps).astype(np.float16)
    say("one-hot", M, K, N)
    C = run_gemm(A, Bq, S, 128)
    C16, _ = oracle.gemm(A, Bq, S, 128)
    assert np.array_equal(C.astype(np.float64), C16.astype(np.float64))


def test_gemm_all_codes_eight_gives_zero():
    A, _, S = make_inputs(17, 2048, 128, 128, seed=3)
    Bq = np.full((2048 // 8, 128), 0x88888888, dtype=np.uint32)
    say("codes eight")
    C = run_gemm(A, Bq, S, 128)
    assert not np.any(C.astype(np.float64))


# ---------------------------------------------------------------------------
# GEMM: random inputs within the bound
# ---------------------------------------------------------------------------

SMALL_CASES = [
    # M, K, N, group: several tiles, ragged M, N not a multiple of 64
    (1, 128, 16, 128), (1, 4096, 4096, 128), (3, 256, 48, 128), (16, 1024, 272, 128),
    (17, 512, 64, 128), (33, 768, 80, 128), (64, 2048, 512, 128), (100, 1024, 208, 256),
    (128, 4096, 1024, 128), (129, 512, 128, 128), (300, 1280, 96, 1280), (513, 256, 64, 128),
    (8, 13824, 160, 13824), (2, 28672, 64, 128),
]


@pytest.mark.parametrize("M,K,N,group", SMALL_CASES)
def test_gemm_matches_oracle(M, K, N, group):
    A, Bq, S = make_inputs(M, K, N, group, seed=M * 31 + K + N)
    say("gemm", M, K, N, group, "workspace", w4.w4a16_workspace_bytes(M, K, N, group))
    C = run_gemm(A, Bq, S, group)
    _, C64 = oracle.gemm(A, Bq, S, group)
    assert_gemm_close(C, C64, f"M={M} K={K} N={N} g={group}")


# Every compiled variant, with and without K splits (fields: mb, nb, wk,
# splits, depth[, tile, unused, wm]; tile 0 the streaming kernel, 2 the LDS
# kernel, whose eighth field is the number of waves along M).
STREAM_PLANS = ["1,1,8,1,2", "1,1,8,3,2", "1,1,8,5,2", "1,2,8,1,2", "1,2,8,4,2",
                "1,4,4,1,2", "1,4,4,7,2", "1,4,4,1,4", "1,4,4,2,4"]
LDS_PLANS = ["1,2,8,1,4,2", "1,2,8,4,4,2", "2,2,8,1,4,2", "2,2,8,8,4,2", "4,1,8,1,3,2",
             "4,1,8,2,3,2", "4,1,8,6,3,2", "8,2,8,1,3,2", "8,2,8,3,3,2"]
LDS_GRID_PLANS = ["4,2,4,1,3,2,0,2", "4,2,4,5,3,2,0,2"]
KERNEL_OF_TILE = {0: "gemm_kernel", 2: "gemm_lds_kernel"}


def _forced_plan_case(monkeypatch, plan, group):
    """M = 45 exercises ragged rows; N = 208 a ragged column tile."""
    M, K, N = 45, 3584, 208
    A, Bq, S = make_inputs(M, K, N, group, seed=5)
    _, C64 = oracle.gemm(A, Bq, S, group)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, group)
    fields = [int(x) for x in plan.split(",")]
    kernel = KERNEL_OF_TILE[fields[5] if len(fields) > 5 else 0]
    assert desc.startswith(kernel + "<"), desc   # the forced variant is the one that runs
    mb, nb, wk, splits, depth = fields[:5]
    if len(fields) > 5 and fields[5] == 2:
        wm = fields[7] if len(fields) > 7 else 1
        assert desc.startswith(f"{kernel}<{mb},{nb},{wm},{wk},{depth}>"), desc
    else:
        assert desc.startswith(f"{kernel}<{mb},{nb},{wk},{depth}>"), desc
    assert f"splits={min(splits, K // 128)} " in desc, desc
    say("forced plan", plan, "group", group, desc)
    C = run_gemm(A, Bq, S, group)
    assert_gemm_close(C, C64, f"plan {plan} group {group}")


@pytest.mark.parametrize("plan", STREAM_PLANS + LDS_PLANS + LDS_GRID_PLANS)
def test_gemm_forced_plans_agree(monkeypatch, plan):
    """Every compiled variant and split count gives the oracle's answer."""
    _forced_plan_case(monkeypatch, plan, 128)


@pytest.mark.parametrize("plan", ["1,2,8,3,2", "1,4,4,2,4", "2,2,8,3,4,2", "8,2,8,2,3,2",
                                  "4,2,4,2,3,2,0,2"])
def test_gemm_forced_plans_coarse_groups(monkeypatch, plan):
    """A scale group of four K blocks (512): each K block finds its group row."""
    _forced_plan_case(monkeypatch, plan, 512)


# Forced split-K plans for the workspace-reuse test: the streaming kernel
# with 16-column tiles and the LDS kernel with 64 x 128 tiles, both split.
REUSE_PLANS = ["1,1,8,2,2", "4,1,8,2,3,2"]


@pytest.mark.parametrize("plan", REUSE_PLANS)
def test_gemm_workspace_reuse_across_shapes(plan):
    """One workspace, zero-filled once, serves split-K calls of two shapes in
    turn: the second shape has more output tiles than the first, so with
    counters placed after the first call's tile count its counters would
    land on the first call's partial sums.  Both outputs match the oracle
    and repeat bit for bit."""
    import torch
    w4.w4a16_set_forced_plan(plan)
    shapes = [(16, 2048, 1024), (16, 2048, 4096)]
    cases = []
    for i, (M, K, N) in enumerate(shapes):
        A, Bq, S = make_inputs(M, K, N, 128, seed=20 + i)
        desc = w4.w4a16_describe(M, K, N, 128)
        assert "splits=1 " not in desc, desc
        cases.append((A, Bq, S, repack_on_device(dev(Bq), K, N), desc))
    tiles = [int(c[4].split("grid=")[1].split("x")[0]) for c in cases]
    assert tiles[1] > tiles[0], tiles
    need = max(w4.w4a16_workspace_bytes(M, K, N, 128) for M, K, N in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    firsts = []
    for (A, Bq, S, Bp, desc) in cases:
        say("workspace reuse", plan, desc)
        C = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
        _, C64 = oracle.gemm(A, Bq, S, 128)
        assert_gemm_close(C, C64, desc)
        firsts.append(C)
    for rnd in range(3):
        for i, (A, Bq, S, Bp, desc) in enumerate(cases):
            again = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
            assert np.array_equal(firsts[i].view(np.uint16), again.view(np.uint16)), \
                f"round {rnd} shape {shapes[i]}"
    # every counter is back at zero after the calls
    torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_gemm_deterministic_repeats():
    """Bit-identical output over repeated calls sharing one workspace, with a
    call of another shape in between."""
    import torch
    M, K, N = 16, 4096, 4096
    A, Bq, S = make_inputs(M, K, N, 128, seed=0)
    A2, Bq2, S2 = make_inputs(3, 2048, 1024, 128, seed=1)
    need = max(w4.w4a16_workspace_bytes(M, K, N, 128), w4.w4a16_workspace_bytes(3, 2048, 1024, 128))
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    Bp = repack_on_device(dev(Bq), K, N)
    say("determinism", M, K, N, "workspace", need)
    first = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
    for i in range(20):
        if i == 10:
            run_gemm(A2, Bq2, S2, 128, workspace=ws)
        again = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
        assert np.array_equal(first.view(np.uint16), again.view(np.uint16)), f"run {i}"
    _, C64 = oracle.gemm(A, Bq, S, 128)
    assert_gemm_close(first, C64)


@pytest.mark.parametrize("M,K,N,plan", [(128, 4096, 4096, "4,1,8,4,3,2"),
                                        (64, 11008, 1024, "4,1,8,4,3,2"),
                                        (300, 2048, 512, "8,2,8,2,3,2")])
def test_lds_kernel_split_k_deterministic(M, K, N, plan):
    """The LDS kernel's split-K path (forced): bit-identical repeats on one
    workspace."""
    import torch
    A, Bq, S = make_inputs(M, K, N, 128, seed=M + K)
    w4.w4a16_set_forced_plan(plan)
    desc = w4.w4a16_describe(M, K, N, 128)
    assert desc.startswith("gemm_lds_kernel<") and "splits=1 " not in desc, desc
    ws = w4.alloc_workspace(M, K, N, 128)
    Bp = repack_on_device(dev(Bq), K, N)
    say("lds determinism", M, K, N, desc)
    first = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
    for i in range(10):
        again = run_gemm(A, Bq, S, 128, workspace=ws, Bp=Bp)
        assert np.array_equal(first.view(np.uint16), again.view(np.uint16)), f"run {i}"
    _, C64 = oracle.gemm(A, Bq, S, 128)
    assert_gemm_close(first, C64)


def test_gemm_empty_m_leaves_output_alone():
    import torch
    K, N = 256, 64
    _, Bq, S = make_inputs(1, K, N, 128)
    Bp = repack_on_device(dev(Bq), K, N)
    C = torch.full((1, N), 7.0, dtype=torch.float16, device="cuda")
    A = torch.zeros((1, K), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm(A, Bp, dev(S), C, 0, K, N, 128, None)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_gemm_rows_beyond_m_untouched():
    """C rows at and past M are never written (C is given extra rows)."""
    import torch
    M, K, N = 5, 512, 64
    A, Bq, S = make_inputs(M, K, N, 128, seed=2)
    Bp = repack_on_device(dev(Bq), K, N)
    C = torch.full((M + 3, N), 7.0, dtype=torch.float16, device="cuda")
    ws = w4.alloc_workspace(M, K, N, 128)
    w4.w4a16_gemm(dev(A), Bp, dev(S), C, M, K, N, 128, ws)
    torch.cuda.synchronize()
    assert torch.all(C[M:] == 7.0)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    assert_gemm_close(host_f16(C[:M]), C64)


def test_gemm_missing_workspace_is_rejected():
    import torch
    M, K, N = 1, 4096, 64       # few tiles and a deep K: the plan splits K
    if w4.w4a16_workspace_bytes(M, K, N, 128) == 0:
        pytest.skip("this shape needs no workspace on this device")
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Bp = w4.alloc_packed(K, N)
    S = torch.ones((K // 128, N), dtype=torch.float16, device="cuda")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm(A, Bp, S, C, M, K, N, 128, None)
    assert e.value.name == "W4A16_ERR_WORKSPACE"


def test_gemm_graph_capture_replays():
    """Captured into a HIP graph, replays match the eager call every time."""
    import torch
    M, K, N = 16, 4096, 1024
    A, Bq, S = make_inputs(M, K, N, 128, seed=4)
    Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    ws = w4.alloc_workspace(M, K, N, 128)
    C_eager = torch.empty((M, N), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm(A_d, Bp, S_d, C_eager, M, K, N, 128, ws)
    torch.cuda.synchronize()
    C_g = torch.empty_like(C_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("graph capture")
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            w4.w4a16_gemm(A_d, Bp, S_d, C_g, M, K, N, 128, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(4):
        C_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C_g.view(torch.int16), C_eager.view(torch.int16)), f"replay {i}"
        w4.w4a16_gemm(A_d, Bp, S_d, C_eager, M, K, N, 128, ws)   # eager work in between
        torch.cuda.synchronize()


def test_workspace_aliasing_an_input_is_rejected():
    """Partial tiles are written while other workgroups read the inputs: a
    workspace overlapping A, the weights or the scales is refused before any
    launch."""
    import ctypes
    import torch
    w4.w4a16_set_forced_plan("1,1,8,2,2")
    M, K, N, g = 16, 2048, 1024, 128
    A, Bq, S = make_inputs(M, K, N, g, seed=3)
    need = w4.w4a16_workspace_bytes(M, K, N, g)
    assert need > 0
    big = torch.zeros(need + M * K * 2, dtype=torch.uint8, device="cuda")
    A_d = big[: M * K * 2].view(torch.float16)
    A_d.copy_(dev(A).view(-1))
    Bp = repack_on_device(dev(Bq), K, N)
    S_d = dev(S)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    lib = w4.load()
    stream = torch.cuda.current_stream().cuda_stream
    for ws_ptr in (A_d.data_ptr(), Bp.data_ptr(), S_d.data_ptr()):
        rc = lib.w4a16_gemm(A_d.data_ptr(), Bp.data_ptr(), S_d.data_ptr(), C.data_ptr(), M, K, N,
                            g, ctypes.c_void_p(ws_ptr), stream)
        assert rc == -2, rc   # W4A16_ERR_SHAPE
    # a separate workspace is accepted
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    w4.w4a16_gemm(A_d, Bp, S_d, C, M, K, N, g, ws)
    torch.cuda.synchronize()


def test_binding_refuses_buffers_too_small():
    """The C interface takes no sizes: the binding checks every tensor's
    bytes before a pointer reaches the library."""
    import torch
    M, K, N, g = 4, 256, 64, 128
    A, Bq, S = make_inputs(M, K, N, g, seed=4)
    Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    short = torch.empty((M - 1, N), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="C"):
        w4.w4a16_gemm(A_d, Bp, S_d, short, M, K, N, g, None)
    with pytest.raises(ValueError, match="A"):
        w4.w4a16_gemm(A_d[:2], Bp, S_d, C, M, K, N, g, None)
    with pytest.raises(ValueError, match="scales"):
        w4.w4a16_gemm(A_d, Bp, S_d[:1, :32].contiguous(), C, M, K, N, g, None)
    with pytest.raises(ValueError, match="Bpacked"):
        w4.w4a16_gemm(A_d, Bp[:16], S_d, C, M, K, N, g, None)
    W = torch.empty((K - 128, N), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="W"):
        w4.w4a16_dequant_debug(Bp, S_d, W, K, N, g)


def test_lds_tail_tiles_split():
    """With more tiles than compute units and a partial last wave, the LDS
    kernel runs the whole waves' tiles whole and splits only the remaining
    ones in K: M = 300 and N = 28672 give 3 x 112 = 336 tiles of 128 x 256,
    256 whole and 80 split.  Matches the oracle everywhere, repeats bit for
    bit, and leaves the counters at zero."""
    import torch
    M, K, N, g = 300, 2048, 28672, 128
    desc = w4.w4a16_describe(M, K, N, g)
    assert desc.startswith("gemm_lds_kernel<") and "whole=256 " in desc, desc
    assert "splits=1 " not in desc, desc
    A, Bq, S = make_inputs(M, K, N, g, seed=30)
    Bp = repack_on_device(dev(Bq), K, N)
    ws = torch.zeros(w4.w4a16_workspace_bytes(M, K, N, g), dtype=torch.uint8, device="cuda")
    say("lds tail split", desc)
    first = run_gemm(A, Bq, S, g, workspace=ws, Bp=Bp)
    again = run_gemm(A, Bq, S, g, workspace=ws, Bp=Bp)
    assert np.array_equal(first.view(np.uint16), again.view(np.uint16))
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    _, C64 = oracle.gemm(A, Bq, S, g)
    assert_gemm_close(first, C64, desc)
