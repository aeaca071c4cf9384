"""MI355X-native W4A16 matmul: Python binding of libw4a16.so.

The binding only marshals arguments: every step of the computation runs in
the library's HIP kernels.  torch provides device memory and the current
stream.  The functions carry the C interface's names (include/w4a16.h):

    w4a16_repack(Bq, Bpacked, K, N, stream=None)
    w4a16_gemm(A, Bpacked, scales, C, M, K, N, group, workspace, stream=None)
    w4a16_gemm_noalloc(A, Bpacked, scales, C, M, K, N, group, stream=None)
    w4a16_gemm_fused(A, Bpacked, scales, bias, activation, C, M, K, N, group,
                     workspace, stream=None)
    w4a16_dequant_debug(Bpacked, scales, W, K, N, group, stream=None)
    w4a16_gemm_awq(A, Bpacked, scales, zeros, C, M, K, N, group, dtype,
                   workspace, stream=None)
    w4a16_dequant_awq_debug(Bpacked, scales, zeros, W, K, N, group, dtype,
                            stream=None)
    w8a16_repack(Bq8, Bpacked, K, N, stream=None)
    w8a16_gemm(A, Bpacked, scales, C, M, K, N, group, workspace, stream=None)
    w8a16_dequant_debug(Bpacked, scales, W, K, N, group, stream=None)
    w8a16_packed_bytes(K, N)
    w8a16_workspace_bytes(M, K, N, group)
    w8a16_describe(M, K, N, group)
    w4a16_sparse24_repack(Bq, mask, Bpacked, K, N, stream=None)
    w4a16_sparse24_gemm(A, Bpacked, scales, C, M, K, N, group, workspace,
                        stream=None)
    w4a16_sparse24_dequant_debug(Bpacked, scales, W, K, N, group, stream=None)
    w4a16_sparse24_packed_bytes(K, N)
    w4a16_sparse24_workspace_bytes(M, K, N, group)
    w4a16_sparse24_describe(M, K, N, group)
    w4a16_workspace_bytes(M, K, N, group)
    w4a16_packed_bytes(K, N)
    w4a16_layout_version()
    w4a16_status_string(status)
    w4a16_set_forced_plan(spec)          (tuning and testing only)

A missing library is an error (``LibraryNotBuilt``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "W4A16Error", "LibraryNotBuilt", "library_path", "load",
    "w4a16_repack", "w4a16_gemm", "w4a16_gemm_fused", "w4a16_dequant_debug",
    "W4A16_ACT_NONE", "W4A16_ACT_RELU", "W4A16_ACT_SILU",
    "w4a16_gemm_awq", "w4a16_dequant_awq_debug", "W4A16_DTYPE_F16", "W4A16_DTYPE_BF16",
    "w8a16_repack", "w8a16_gemm", "w8a16_dequant_debug", "w8a16_packed_bytes",
    "w8a16_workspace_bytes", "w8a16_describe", "alloc_workspace8",
    "w4a16_sparse24_repack", "w4a16_sparse24_gemm", "w4a16_sparse24_dequant_debug",
    "w4a16_sparse24_packed_bytes", "w4a16_sparse24_workspace_bytes", "w4a16_sparse24_describe",
    "w4a16_workspace_bytes", "w4a16_packed_bytes", "w4a16_layout_version",
    "w4a16_status_string", "w4a16_describe", "w4a16_plan_describe", "w4a16_set_forced_plan",
    "w4a16_gemm_noalloc",
    "W4A16_NOALLOC_SCRATCH_BYTES", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libw4a16.so"

# Status codes and activations of include/w4a16.h.
W4A16_OK = 0
W4A16_ACT_NONE = 0
W4A16_ACT_RELU = 1
W4A16_ACT_SILU = 2
W4A16_DTYPE_F16 = 0
W4A16_DTYPE_BF16 = 1
W4A16_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

EXPORTED_SYMBOLS = (
    "w4a16_layout_version", "w4a16_status_string", "w4a16_packed_bytes",
    "w4a16_workspace_bytes", "w4a16_repack", "w4a16_gemm", "w4a16_dequant_debug",
    "w4a16_describe", "w4a16_gemm_fused", "w4a16_gemm_awq", "w4a16_dequant_awq_debug",
    "w8a16_packed_bytes", "w8a16_repack", "w8a16_gemm", "w8a16_dequant_debug",
    "w4a16_sparse24_packed_bytes", "w4a16_sparse24_repack", "w4a16_sparse24_workspace_bytes",
    "w4a16_sparse24_describe", "w4a16_sparse24_gemm", "w4a16_sparse24_dequant_debug",
    "w4a16_set_forced_plan", "w4a16_gemm_noalloc", "w8a16_workspace_bytes", "w8a16_describe",
    "w4a16_plan_describe",
)


class LibraryNotBuilt(RuntimeError):
    pass


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, status: int, name: str):
        super().__init__(f"{fn} failed: {name} ({status})")
        self.status = status
        self.name = name


def library_path() -> str:
    return os.environ.get("W4A16_LIBRARY", os.path.join(_PKG, _LIB_NAME))


_lib = None


def load():
    """Load libw4a16.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} not found; build it with `python -m weight_only_int4_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.w4a16_layout_version.argtypes = []
    lib.w4a16_layout_version.restype = i
    lib.w4a16_status_string.argtypes = [i]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_packed_bytes.argtypes = [i, i]
    lib.w4a16_packed_bytes.restype = sz
    lib.w4a16_workspace_bytes.argtypes = [i, i, i, i]
    lib.w4a16_workspace_bytes.restype = sz
    lib.w4a16_repack.argtypes = [vp, vp, i, i, vp]
    lib.w4a16_repack.restype = i
    lib.w4a16_gemm.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp]
    lib.w4a16_gemm.restype = i
    lib.w4a16_gemm_fused.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, vp, vp]
    lib.w4a16_gemm_fused.restype = i
    lib.w4a16_gemm_awq.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    lib.w4a16_gemm_awq.restype = i
    lib.w4a16_dequant_awq_debug.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.w4a16_dequant_awq_debug.restype = i
    lib.w8a16_packed_bytes.argtypes = [i, i]
    lib.w8a16_packed_bytes.restype = sz
    lib.w8a16_repack.argtypes = [vp, vp, i, i, vp]
    lib.w8a16_repack.restype = i
    lib.w8a16_workspace_bytes.argtypes = [i, i, i, i]
    lib.w8a16_workspace_bytes.restype = sz
    lib.w8a16_describe.argtypes = [i, i, i, i, ctypes.c_char_p, sz]
    lib.w8a16_describe.restype = i
    lib.w8a16_gemm.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp]
    lib.w8a16_gemm.restype = i
    lib.w8a16_dequant_debug.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.w8a16_dequant_debug.restype = i
    lib.w4a16_dequant_debug.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.w4a16_dequant_debug.restype = i
    lib.w4a16_describe.argtypes = [i, i, i, i, ctypes.c_char_p, sz]
    lib.w4a16_describe.restype = i
    lib.w4a16_plan_describe.argtypes = [i, i, i, i, i, i, ctypes.c_char_p, sz]
    lib.w4a16_plan_describe.restype = i
    lib.w4a16_sparse24_packed_bytes.argtypes = [i, i]
    lib.w4a16_sparse24_packed_bytes.restype = sz
    lib.w4a16_sparse24_repack.argtypes = [vp, vp, vp, i, i, vp]
    lib.w4a16_sparse24_repack.restype = i
    lib.w4a16_sparse24_workspace_bytes.argtypes = [i, i, i, i]
    lib.w4a16_sparse24_workspace_bytes.restype = sz
    lib.w4a16_sparse24_describe.argtypes = [i, i, i, i, ctypes.c_char_p, sz]
    lib.w4a16_sparse24_describe.restype = i
    lib.w4a16_sparse24_gemm.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp]
    lib.w4a16_sparse24_gemm.restype = i
    lib.w4a16_sparse24_dequant_debug.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.w4a16_sparse24_dequant_debug.restype = i
    lib.w4a16_gemm_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.w4a16_gemm_noalloc.restype = i
    lib.w4a16_set_forced_plan.argtypes = [ctypes.c_char_p]
    lib.w4a16_set_forced_plan.restype = i
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    """Device address of a tensor (or None / a raw int address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != W4A16_OK:
        raise W4A16Error(fn, status, w4a16_status_string(status))


def _expect(t, dtype, what):
    if t is None or isinstance(t, int):
        return
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a device tensor")


def _need(t, nbytes: int, what: str):
    """The C interface takes no buffer sizes: a tensor smaller than the call
    reads or writes, or one on another device than the current one, is
    refused here, before any pointer reaches the library."""
    if t is None or isinstance(t, int):
        return
    import torch
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, the call needs {nbytes}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what}: on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _shape_ok(M: int, K: int, N: int, group: int) -> bool:
    """Shapes whose buffer sizes are defined; the library rejects the rest
    with its own status code."""
    return M >= 0 and K > 0 and N >= 0 and group > 0 and K % group == 0


def _need_gemm(M, K, N, group, A, Bpacked, packed_bytes, scales, C, workspace, ws_bytes,
               zeros=None, bias=None):
    M, K, N, group = int(M), int(K), int(N), int(group)
    if not _shape_ok(M, K, N, group) or M == 0 or N == 0:
        return
    _need(A, M * K * 2, "A")
    _need(Bpacked, packed_bytes, "Bpacked")
    _need(scales, (K // group) * N * 2, "scales")
    _need(zeros, (K // group) * N, "zeros")
    _need(bias, N * 2, "bias")
    _need(C, M * N * 2, "C")
    if ws_bytes:
        _need(workspace, ws_bytes, "workspace")


def _need_weights(K, N, group, Bpacked, packed_bytes, scales, W, zeros=None):
    K, N, group = int(K), int(N), int(group)
    if not _shape_ok(0, K, N, group) or N == 0:
        return
    _need(Bpacked, packed_bytes, "Bpacked")
    _need(scales, (K // group) * N * 2, "scales")
    _need(zeros, (K // group) * N, "zeros")
    _need(W, K * N * 2, "W")


# ---------------------------------------------------------------------------
# the C interface, name for name
# ---------------------------------------------------------------------------

def w4a16_layout_version() -> int:
    return load().w4a16_layout_version()


def w4a16_status_string(status: int) -> str:
    return load().w4a16_status_string(int(status)).decode()


def w4a16_packed_bytes(K: int, N: int) -> int:
    return load().w4a16_packed_bytes(int(K), int(N))


def w4a16_workspace_bytes(M: int, K: int, N: int, group: int) -> int:
    return load().w4a16_workspace_bytes(int(M), int(K), int(N), int(group))


def w4a16_describe(M: int, K: int, N: int, group: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check("w4a16_describe", load().w4a16_describe(int(M), int(K), int(N), int(group), buf, 256))
    return buf.value.decode()


# weight formats of w4a16_plan_describe (enum w4a16_format)
W4A16_FORMAT_F16, W4A16_FORMAT_F16_ZP, W4A16_FORMAT_BF16, W4A16_FORMAT_BF16_ZP = 0, 1, 2, 3
W4A16_FORMAT_W8, W4A16_FORMAT_SPARSE24 = 4, 5


def w4a16_plan_describe(M: int, K: int, N: int, group: int, fmt: int, cus: int) -> str:
    """The plan of a call of weight format ``fmt`` on a device with ``cus``
    compute units, computed without a device."""
    buf = ctypes.create_string_buffer(256)
    _check("w4a16_plan_describe", load().w4a16_plan_describe(int(M), int(K), int(N), int(group),
                                                             int(fmt), int(cus), buf, 256))
    return buf.value.decode()


def w4a16_set_forced_plan(spec=None) -> None:
    """Tuning and testing only: force the plan of later calls (see the
    header for the text); None restores the heuristic."""
    arg = None if not spec else str(spec).encode()
    _check("w4a16_set_forced_plan", load().w4a16_set_forced_plan(arg))


def w4a16_repack(Bq, Bpacked, K: int, N: int, stream=None) -> None:
    import torch
    _expect(Bq, torch.int32, "Bq")
    _expect(Bpacked, torch.int32, "Bpacked")
    if int(K) > 0 and int(N) > 0:
        _need(Bq, int(K) * int(N) // 2, "Bq")
        _need(Bpacked, w4a16_packed_bytes(K, N), "Bpacked")
    _check("w4a16_repack", load().w4a16_repack(_ptr(Bq), _ptr(Bpacked), int(K), int(N),
                                               _stream(stream)))


def w4a16_gemm(A, Bpacked, scales, C, M: int, K: int, N: int, group: int,
               workspace=None, stream=None) -> None:
    import torch
    _expect(A, torch.float16, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(C, torch.float16, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w4a16_packed_bytes(K, N), scales, C, workspace,
               w4a16_workspace_bytes(M, K, N, group))
    _check("w4a16_gemm", load().w4a16_gemm(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(C),
                                           int(M), int(K), int(N), int(group),
                                           _ptr(workspace), _stream(stream)))


def w4a16_gemm_noalloc(A, Bpacked, scales, C, M: int, K: int, N: int, group: int,
                       stream=None) -> None:
    """w4a16_gemm with the library's own per-device scratch: no workspace."""
    import torch
    _expect(A, torch.float16, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(C, torch.float16, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w4a16_packed_bytes(K, N), scales, C, None, 0)
    _check("w4a16_gemm_noalloc",
           load().w4a16_gemm_noalloc(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(C), int(M),
                                     int(K), int(N), int(group), _stream(stream)))


def w4a16_gemm_fused(A, Bpacked, scales, bias, activation: int, C, M: int, K: int, N: int,
                     group: int, workspace=None, stream=None) -> None:
    import torch
    _expect(A, torch.float16, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(bias, torch.float16, "bias")
    _expect(C, torch.float16, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w4a16_packed_bytes(K, N), scales, C, workspace,
               w4a16_workspace_bytes(M, K, N, group), bias=bias)
    _check("w4a16_gemm_fused",
           load().w4a16_gemm_fused(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(bias),
                                   int(activation), _ptr(C), int(M), int(K), int(N),
                                   int(group), _ptr(workspace), _stream(stream)))


def _expect16(t, what):
    """A 16-bit tensor: float16, or BF16 passed as bfloat16 / int16 bits."""
    import torch
    if t is None or isinstance(t, int):
        return
    if t.dtype not in (torch.float16, torch.bfloat16, torch.int16):
        raise TypeError(f"{what}: expected a 16-bit tensor, got {t.dtype}")
    _expect(t, t.dtype, what)


def w4a16_gemm_awq(A, Bpacked, scales, zeros, C, M: int, K: int, N: int, group: int,
                   dtype: int, workspace=None, stream=None) -> None:
    import torch
    _expect16(A, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect16(scales, "scales")
    _expect(zeros, torch.uint8, "zeros")
    _expect16(C, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w4a16_packed_bytes(K, N), scales, C, workspace,
               w4a16_workspace_bytes(M, K, N, group), zeros=zeros)
    _check("w4a16_gemm_awq",
           load().w4a16_gemm_awq(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(zeros), _ptr(C),
                                 int(M), int(K), int(N), int(group), int(dtype),
                                 _ptr(workspace), _stream(stream)))


def w4a16_dequant_awq_debug(Bpacked, scales, zeros, W, K: int, N: int, group: int, dtype: int,
                            stream=None) -> None:
    import torch
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect16(scales, "scales")
    _expect(zeros, torch.uint8, "zeros")
    _expect16(W, "W")
    _need_weights(K, N, group, Bpacked, w4a16_packed_bytes(K, N), scales, W, zeros=zeros)
    _check("w4a16_dequant_awq_debug",
           load().w4a16_dequant_awq_debug(_ptr(Bpacked), _ptr(scales), _ptr(zeros), _ptr(W),
                                          int(K), int(N), int(group), int(dtype),
                                          _stream(stream)))


def w8a16_packed_bytes(K: int, N: int) -> int:
    return load().w8a16_packed_bytes(int(K), int(N))


def w8a16_workspace_bytes(M: int, K: int, N: int, group: int) -> int:
    return load().w8a16_workspace_bytes(int(M), int(K), int(N), int(group))


def w8a16_describe(M: int, K: int, N: int, group: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check("w8a16_describe", load().w8a16_describe(int(M), int(K), int(N), int(group), buf, 256))
    return buf.value.decode()


def w8a16_repack(Bq8, Bpacked, K: int, N: int, stream=None) -> None:
    import torch
    _expect(Bq8, torch.int32, "Bq8")
    _expect(Bpacked, torch.int32, "Bpacked")
    if int(K) > 0 and int(N) > 0:
        _need(Bq8, int(K) * int(N), "Bq8")
        _need(Bpacked, w8a16_packed_bytes(K, N), "Bpacked")
    _check("w8a16_repack", load().w8a16_repack(_ptr(Bq8), _ptr(Bpacked), int(K), int(N),
                                               _stream(stream)))


def w8a16_gemm(A, Bpacked, scales, C, M: int, K: int, N: int, group: int,
               workspace=None, stream=None) -> None:
    import torch
    _expect(A, torch.float16, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(C, torch.float16, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w8a16_packed_bytes(K, N), scales, C, workspace,
               w8a16_workspace_bytes(M, K, N, group))
    _check("w8a16_gemm", load().w8a16_gemm(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(C),
                                           int(M), int(K), int(N), int(group),
                                           _ptr(workspace), _stream(stream)))


def w8a16_dequant_debug(Bpacked, scales, W, K: int, N: int, group: int, stream=None) -> None:
    import torch
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(W, torch.float16, "W")
    _need_weights(K, N, group, Bpacked, w8a16_packed_bytes(K, N), scales, W)
    _check("w8a16_dequant_debug",
           load().w8a16_dequant_debug(_ptr(Bpacked), _ptr(scales), _ptr(W), int(K), int(N),
                                      int(group), _stream(stream)))


def w4a16_dequant_debug(Bpacked, scales, W, K: int, N: int, group: int,
                        stream=None) -> None:
    import torch
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(W, torch.float16, "W")
    _need_weights(K, N, group, Bpacked, w4a16_packed_bytes(K, N), scales, W)
    _check("w4a16_dequant_debug",
           load().w4a16_dequant_debug(_ptr(Bpacked), _ptr(scales), _ptr(W), int(K), int(N),
                                      int(group), _stream(stream)))


def w4a16_sparse24_packed_bytes(K: int, N: int) -> int:
    return load().w4a16_sparse24_packed_bytes(int(K), int(N))


def w4a16_sparse24_workspace_bytes(M: int, K: int, N: int, group: int) -> int:
    return load().w4a16_sparse24_workspace_bytes(int(M), int(K), int(N), int(group))


def w4a16_sparse24_describe(M: int, K: int, N: int, group: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check("w4a16_sparse24_describe",
           load().w4a16_sparse24_describe(int(M), int(K), int(N), int(group), buf, 256))
    return buf.value.decode()


def w4a16_sparse24_repack(Bq, mask, Bpacked, K: int, N: int, stream=None) -> None:
    import torch
    _expect(Bq, torch.int32, "Bq")
    _expect(mask, torch.uint8, "mask")
    _expect(Bpacked, torch.int32, "Bpacked")
    if int(K) > 0 and int(N) > 0:
        _need(Bq, int(K) * int(N) // 2, "Bq")
        _need(mask, int(K) * int(N) // 4, "mask")
        _need(Bpacked, w4a16_sparse24_packed_bytes(K, N), "Bpacked")
    _check("w4a16_sparse24_repack",
           load().w4a16_sparse24_repack(_ptr(Bq), _ptr(mask), _ptr(Bpacked), int(K), int(N),
                                        _stream(stream)))


def w4a16_sparse24_gemm(A, Bpacked, scales, C, M: int, K: int, N: int, group: int,
                        workspace=None, stream=None) -> None:
    import torch
    _expect(A, torch.float16, "A")
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(C, torch.float16, "C")
    _need_gemm(M, K, N, group, A, Bpacked, w4a16_sparse24_packed_bytes(K, N), scales, C,
               workspace, w4a16_sparse24_workspace_bytes(M, K, N, group))
    _check("w4a16_sparse24_gemm",
           load().w4a16_sparse24_gemm(_ptr(A), _ptr(Bpacked), _ptr(scales), _ptr(C), int(M),
                                      int(K), int(N), int(group), _ptr(workspace),
                                      _stream(stream)))


def w4a16_sparse24_dequant_debug(Bpacked, scales, W, K: int, N: int, group: int,
                                 stream=None) -> None:
    import torch
    _expect(Bpacked, torch.int32, "Bpacked")
    _expect(scales, torch.float16, "scales")
    _expect(W, torch.float16, "W")
    _need_weights(K, N, group, Bpacked, w4a16_sparse24_packed_bytes(K, N), scales, W)
    _check("w4a16_sparse24_dequant_debug",
           load().w4a16_sparse24_dequant_debug(_ptr(Bpacked), _ptr(scales), _ptr(W), int(K),
                                               int(N), int(group), _stream(stream)))


# ---------------------------------------------------------------------------
# allocation conveniences (torch owns the memory; the library allocates none)
# ---------------------------------------------------------------------------

def alloc_workspace(M: int, K: int, N: int, group: int, device=None):
    """A zero-filled workspace of ``w4a16_workspace_bytes`` bytes, or None."""
    import torch
    nbytes = w4a16_workspace_bytes(M, K, N, group)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device or "cuda")


def alloc_workspace8(M: int, K: int, N: int, group: int, device=None):
    """A zero-filled workspace of ``w8a16_workspace_bytes`` bytes, or None."""
    import torch
    nbytes = w8a16_workspace_bytes(M, K, N, group)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device or "cuda")


def alloc_packed(K: int, N: int, device=None):
    """An int32 tensor of ``w4a16_packed_bytes(K, N)`` bytes for repacked codes."""
    import torch
    return torch.empty(K * N // 8, dtype=torch.int32, device=device or "cuda")


def alloc_packed8(K: int, N: int, device=None):
    """An int32 tensor of ``w8a16_packed_bytes(K, N)`` bytes for repacked 8-bit codes."""
    import torch
    return torch.empty(K * N // 4, dtype=torch.int32, device=device or "cuda")


def alloc_packed_sparse24(K: int, N: int, device=None):
    """An int32 tensor of ``w4a16_sparse24_packed_bytes(K, N)`` bytes for 2:4 codes."""
    import torch
    return torch.empty(K * N * 3 // 32, dtype=torch.int32, device=device or "cuda")


def alloc_workspace_sparse24(M: int, K: int, N: int, group: int, device=None):
    """A zero-filled workspace of ``w4a16_sparse24_workspace_bytes`` bytes, or None."""
    import torch
    nbytes = w4a16_sparse24_workspace_bytes(M, K, N, group)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device or "cuda")
