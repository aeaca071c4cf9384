"""The allocation-free entry point, w4a16_gemm_noalloc, through the C
interface: on split-K plans (so the library's per-device scratch is used) it
gives exactly what w4a16_gemm gives with a caller's workspace -- the same
plan, the same kernels, the same order of additions -- on two calls in a
row, the second with a smaller input; and it refuses a plan whose partials
exceed the scratch."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import weight_only_int4_gemm_amd as w4
from synth import make_inputs
from tests.gpu_util import dev, repack_on_device, say
from tests.tolerance import assert_gemm_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_plan():
    w4.w4a16_set_forced_plan(None)
    yield
    w4.w4a16_set_forced_plan(None)


def _both(M, K, N, g, seed):
    """(noalloc output, w4a16_gemm output, oracle float64 product)."""
    import torch
    A, Bq, S = make_inputs(M, K, N, g, seed=seed)
    Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    desc = w4.w4a16_describe(M, K, N, g)
    need = w4.w4a16_workspace_bytes(M, K, N, g)
    say("noalloc", M, K, N, g, desc)
    C1 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm_noalloc(A_d, Bp, S_d, C1, M, K, N, g)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    C2 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm(A_d, Bp, S_d, C2, M, K, N, g, ws)
    torch.cuda.synchronize()
    _, C64 = oracle.gemm(A, Bq, S, g)
    return C1.cpu().numpy(), C2.cpu().numpy(), C64, desc, need


# (forced plan, larger shape, smaller shape): the streaming kernel, the
# LDS kernel and the stream-K kernel (five workgroups, so runs share tiles),
# each passing partials through the scratch.
CASES = [
    ("1,1,8,2,2", (16, 2048, 4096), (3, 1024, 1024)),
    ("4,1,8,2,3,2", (96, 2048, 2048), (40, 1024, 512)),
    ("2,4,8,5,3,4", (64, 2048, 2048), (20, 1024, 512)),
    (None, (16, 11008, 4096), (1, 4096, 4096)),
]


@pytest.mark.parametrize("plan,big,small", CASES)
def test_noalloc_matches_the_workspace_entry_point(plan, big, small):
    w4.w4a16_set_forced_plan(plan)
    for i, (M, K, N) in enumerate((big, small)):
        C1, C2, C64, desc, need = _both(M, K, N, 128, seed=40 + i)
        if plan is not None:
            assert "splits=1 " not in desc and need > 0, desc
        assert need <= w4.W4A16_NOALLOC_SCRATCH_BYTES
        assert np.array_equal(C1.view(np.uint16), C2.view(np.uint16)), (M, K, N, desc)
        assert_gemm_close(C1, C64, desc)


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    import torch
    # 128 x 256 tiles split eight ways on a 4096 x 22016 layer: 86 tiles x 8
    # x 128 KiB of partials, past the 64 MiB scratch
    w4.w4a16_set_forced_plan("8,2,8,8,3,2")
    M, K, N, g = 128, 4096, 22016, 128
    need = w4.w4a16_workspace_bytes(M, K, N, g)
    desc = w4.w4a16_describe(M, K, N, g)
    assert need > w4.W4A16_NOALLOC_SCRATCH_BYTES, (need, desc)
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Bp = w4.alloc_packed(K, N)
    S = torch.zeros((K // g, N), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm_noalloc(A, Bp, S, C, M, K, N, g)
    assert e.value.name == "W4A16_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((C == 3.0).all())   # nothing launched
