"""Helpers for the GPU tests: move seeded inputs to the device and run the
library through its C interface."""

from __future__ import annotations

import sys

import numpy as np

import weight_only_int4_gemm_amd as w4


def say(*args):
    """Name the case before a GPU step, flushed, so a failure can be placed."""
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray):
    import torch
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    if x.dtype == np.uint16:          # BF16 bit patterns travel as int16
        x = x.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def host_f16(t) -> np.ndarray:
    return t.cpu().numpy()


def repack_on_device(Bq_d, K: int, N: int):
    Bp = w4.alloc_packed(K, N)
    w4.w4a16_repack(Bq_d, Bp, K, N)
    return Bp


def run_gemm(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int,
             workspace=None, Bp=None):
    """C (numpy float16) = the library's product on the given host inputs."""
    import torch
    M, K = A.shape
    N = Bq.shape[1]
    if Bp is None:
        Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    C_d = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ws = workspace if workspace is not None else w4.alloc_workspace(M, K, N, group)
    w4.w4a16_gemm(A_d, Bp, S_d, C_d, M, K, N, group, ws)
    torch.cuda.synchronize()
    return host_f16(C_d)


def run_gemm_fused(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int, bias, act: int,
                   workspace=None, Bp=None):
    """C (numpy float16) = act(A . dequant(B) + bias) from the library's fused
    entry point; ``bias`` None passes a NULL bias."""
    import torch
    M, K = A.shape
    N = Bq.shape[1]
    if Bp is None:
        Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    b_d = None if bias is None else dev(bias)
    C_d = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ws = workspace if workspace is not None else w4.alloc_workspace(M, K, N, group)
    w4.w4a16_gemm_fused(A_d, Bp, S_d, b_d, act, C_d, M, K, N, group, ws)
    torch.cuda.synchronize()
    return host_f16(C_d)


def host_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_gemm_awq(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, Z, group: int, dtype: int,
                 workspace=None, Bp=None):
    """C as uint16 bits (BF16) or float16 (FP16) from w4a16_gemm_awq."""
    import torch
    M, K = A.shape
    N = Bq.shape[1]
    if Bp is None:
        Bp = repack_on_device(dev(Bq), K, N)
    A_d, S_d = dev(A), dev(S)
    Z_d = None if Z is None else torch.from_numpy(np.ascontiguousarray(Z)).cuda()
    C_d = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    ws = workspace if workspace is not None else w4.alloc_workspace(M, K, N, group)
    w4.w4a16_gemm_awq(A_d, Bp, S_d, Z_d, C_d, M, K, N, group, dtype, ws)
    torch.cuda.synchronize()
    C = host_u16(C_d)
    return C if dtype else C.view(np.float16)


def repack8_on_device(Bq8_d, K: int, N: int):
    Bp = w4.alloc_packed8(K, N)
    w4.w8a16_repack(Bq8_d, Bp, K, N)
    return Bp


def run_gemm8(A: np.ndarray, Bq8: np.ndarray, S: np.ndarray, group: int, workspace=None,
              Bp=None):
    """C (numpy float16) from w8a16_gemm on the given host inputs."""
    import torch
    M, K = A.shape
    N = Bq8.shape[1]
    if Bp is None:
        Bp = repack8_on_device(dev(Bq8), K, N)
    A_d, S_d = dev(A), dev(S)
    C_d = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ws = workspace if workspace is not None else w4.alloc_workspace8(M, K, N, group)
    w4.w8a16_gemm(A_d, Bp, S_d, C_d, M, K, N, group, ws)
    torch.cuda.synchronize()
    return host_f16(C_d)


def repack_sp24_on_device(Bq_d, mask_d, K: int, N: int):
    Bp = w4.alloc_packed_sparse24(K, N)
    w4.w4a16_sparse24_repack(Bq_d, mask_d, Bp, K, N)
    return Bp


def run_gemm_sp24(A: np.ndarray, Bq: np.ndarray, mask: np.ndarray, S: np.ndarray, group: int,
                  workspace=None, Bp=None):
    """C (numpy float16) from w4a16_sparse24_gemm on the given host inputs."""
    import torch
    M, K = A.shape
    N = Bq.shape[1]
    if Bp is None:
        Bp = repack_sp24_on_device(dev(Bq), dev(mask), K, N)
    A_d, S_d = dev(A), dev(S)
    C_d = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ws = workspace if workspace is not None else w4.alloc_workspace_sparse24(M, K, N, group)
    w4.w4a16_sparse24_gemm(A_d, Bp, S_d, C_d, M, K, N, group, ws)
    torch.cuda.synchronize()
    return host_f16(C_d)
