"""The C interface on the CPU: the library loads, exports what the header
declares, and rejects bad arguments before touching the device.

Only host logic is called here (argument checks that return before any HIP
call, and pure helpers); no kernel runs.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import weight_only_int4_gemm_amd as w4
from weight_only_int4_gemm_amd import roofline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_ALIGN = 0, -1, -2, -3, -4
ERR_EPILOGUE = -8
ERR_DTYPE = -9

# Fake, 16-byte aligned addresses: the checks below return before any of
# them is dereferenced or handed to the runtime.
P_A, P_B, P_S, P_C, P_W = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
P_BIAS = 0x60000000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w[48]a16_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return w4.load()


def test_header_declares_the_interface():
    names = _declared_functions()
    assert names == sorted(w4.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_binding_has_the_same_names():
    for name in _declared_functions():
        assert callable(getattr(w4, name)), name


def test_pure_helpers(lib):
    assert w4.w4a16_layout_version() == 1
    assert w4.w4a16_status_string(0) == "W4A16_OK"
    assert w4.w4a16_status_string(-5) == "W4A16_ERR_WORKSPACE"
    assert w4.w4a16_status_string(123) == "W4A16_ERR_UNKNOWN"
    assert w4.w4a16_packed_bytes(4096, 4096) == 4096 * 4096 // 2
    assert w4.w4a16_packed_bytes(0, 16) == 0


def test_layout_version_matches_the_oracle_description():
    import oracle
    assert w4.w4a16_layout_version() == oracle.LAYOUT_VERSION


@pytest.mark.parametrize("K,N,group,expect", [
    (100, 64, 128, ERR_SHAPE),      # K not a multiple of 128
    (0, 64, 128, ERR_SHAPE),
    (-128, 64, 128, ERR_SHAPE),
    (256, 24, 128, ERR_SHAPE),      # N not a multiple of 16
    (256, -16, 128, ERR_SHAPE),
    (256, 64, 64, ERR_GROUP),       # group not a multiple of 128
    (384, 64, 256, ERR_GROUP),      # group does not divide K
    (256, 64, 0, ERR_GROUP),
])
def test_gemm_rejects_bad_shapes(lib, K, N, group, expect):
    rc = lib.w4a16_gemm(P_A, P_B, P_S, P_C, 4, K, N, group, None, None)
    assert rc == expect


def test_gemm_rejects_bad_pointers(lib):
    assert lib.w4a16_gemm(None, P_B, P_S, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert lib.w4a16_gemm(P_A, None, P_S, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert lib.w4a16_gemm(P_A, P_B, None, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert lib.w4a16_gemm(P_A, P_B, P_S, None, 4, 256, 64, 128, None, None) == ERR_NULL
    assert lib.w4a16_gemm(P_A + 8, P_B, P_S, P_C, 4, 256, 64, 128, None, None) == ERR_ALIGN
    assert lib.w4a16_gemm(P_A, P_B, P_S, P_C + 2, 4, 256, 64, 128, None, None) == ERR_ALIGN
    assert lib.w4a16_gemm(P_A, P_B, P_S, P_C, -1, 256, 64, 128, None, None) == ERR_SHAPE
    # C overlapping an input
    assert lib.w4a16_gemm(P_A, P_B, P_S, P_A, 4, 256, 64, 128, None, None) == ERR_SHAPE


def test_gemm_empty_output_is_a_no_op(lib):
    # M == 0 or N == 0: nothing to compute, nothing launched, NULLs allowed
    assert lib.w4a16_gemm(None, None, None, None, 0, 256, 64, 128, None, None) == OK
    assert lib.w4a16_gemm(None, None, None, None, 5, 256, 0, 128, None, None) == OK


def test_gemm_fused_rejects_bad_arguments(lib):
    f = lib.w4a16_gemm_fused
    assert w4.w4a16_status_string(ERR_EPILOGUE) == "W4A16_ERR_EPILOGUE"
    for act in (-1, 3, 100):
        assert f(P_A, P_B, P_S, P_BIAS, act, P_C, 4, 256, 64, 128, None, None) == ERR_EPILOGUE
    # the plain checks still apply, in the same order as w4a16_gemm's
    assert f(P_A, P_B, P_S, P_BIAS, 2, P_C, 4, 100, 64, 128, None, None) == ERR_SHAPE
    assert f(P_A, P_B, P_S, P_BIAS, 2, P_C, 4, 256, 64, 64, None, None) == ERR_GROUP
    assert f(None, P_B, P_S, P_BIAS, 1, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert f(P_A, P_B, P_S, P_BIAS + 2, 1, P_C, 4, 256, 64, 128, None, None) == ERR_ALIGN
    # C overlapping the bias
    assert f(P_A, P_B, P_S, P_C + 64, 0, P_C, 4, 256, 64, 128, None, None) == ERR_SHAPE
    # empty output: nothing to do, the bias may be NULL or not
    assert f(None, None, None, None, 2, None, 0, 256, 64, 128, None, None) == OK
    assert f(None, None, None, P_BIAS, 1, None, 4, 256, 0, 128, None, None) == OK
    # constants of the binding and the header agree
    text = open(HEADER).read()
    for name in ("W4A16_ACT_NONE", "W4A16_ACT_RELU", "W4A16_ACT_SILU"):
        value = int(re.search(name + r"\s*=\s*(\d+)", text).group(1))
        assert getattr(w4, name) == value, name


def test_awq_entry_points_reject_bad_arguments(lib):
    g, d = lib.w4a16_gemm_awq, lib.w4a16_dequant_awq_debug
    P_Z = 0x70000000
    assert w4.w4a16_status_string(ERR_DTYPE) == "W4A16_ERR_DTYPE"
    for dt in (-1, 2, 7):
        assert g(P_A, P_B, P_S, P_Z, P_C, 4, 256, 64, 128, dt, None, None) == ERR_DTYPE
        assert d(P_B, P_S, P_Z, P_W, 256, 64, 128, dt, None) == ERR_DTYPE
    for dt in (0, 1):
        assert g(P_A, P_B, P_S, P_Z, P_C, 4, 100, 64, 128, dt, None, None) == ERR_SHAPE
        assert g(P_A, P_B, P_S, P_Z, P_C, 4, 256, 64, 96, dt, None, None) == ERR_GROUP
        assert g(None, P_B, P_S, P_Z, P_C, 4, 256, 64, 128, dt, None, None) == ERR_NULL
        assert g(P_A, P_B, P_S, P_Z + 4, P_C, 4, 256, 64, 128, dt, None, None) == ERR_ALIGN
        # C overlapping the zero points
        assert g(P_A, P_B, P_S, P_C + 256, P_C, 4, 256, 64, 128, dt, None, None) == ERR_SHAPE
        assert g(None, None, None, None, None, 0, 256, 64, 128, dt, None, None) == OK
        assert d(None, P_S, P_Z, P_W, 256, 64, 128, dt, None) == ERR_NULL
        assert d(P_B, P_S, P_Z + 8, P_W, 256, 64, 128, dt, None) == ERR_ALIGN
        assert d(P_B, P_S, P_Z, P_W, 256, 64, 96, dt, None) == ERR_GROUP
    text = open(HEADER).read()
    for name in ("W4A16_DTYPE_F16", "W4A16_DTYPE_BF16"):
        value = int(re.search(name + r"\s*=\s*(\d+)", text).group(1))
        assert getattr(w4, name) == value, name


def test_w8a16_entry_points(lib):
    assert w4.w8a16_packed_bytes(4096, 4096) == 4096 * 4096
    assert w4.w8a16_packed_bytes(0, 16) == 0
    assert lib.w8a16_repack(None, P_B, 256, 64, None) == ERR_NULL
    assert lib.w8a16_repack(P_A, P_B, 200, 64, None) == ERR_SHAPE
    assert lib.w8a16_repack(P_A + 4, P_B, 256, 64, None) == ERR_ALIGN
    assert lib.w8a16_repack(P_A, P_A + 1024, 256, 64, None) == ERR_SHAPE   # overlap (K*N bytes)
    assert lib.w8a16_gemm(P_A, P_B, P_S, P_C, 4, 100, 64, 128, None, None) == ERR_SHAPE
    assert lib.w8a16_gemm(P_A, P_B, P_S, P_C, 4, 256, 64, 96, None, None) == ERR_GROUP
    assert lib.w8a16_gemm(None, P_B, P_S, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert lib.w8a16_gemm(P_A, P_B, P_S, P_C + 2, 4, 256, 64, 128, None, None) == ERR_ALIGN
    # C overlapping the 8-bit codes (K*N bytes, twice the 4-bit size)
    assert lib.w8a16_gemm(P_A, P_B, P_S, P_B + 256 * 64 - 64, 4, 256, 64, 128, None,
                          None) == ERR_SHAPE
    assert lib.w8a16_gemm(None, None, None, None, 0, 256, 64, 128, None, None) == OK
    assert lib.w8a16_dequant_debug(None, P_S, P_W, 256, 64, 128, None) == ERR_NULL
    assert lib.w8a16_dequant_debug(P_B, P_S, P_W, 256, 64, 96, None) == ERR_GROUP


def test_sparse24_entry_points(lib):
    P_MASK = 0x70000000
    assert w4.w4a16_sparse24_packed_bytes(4096, 4096) == 4096 * 4096 * 3 // 8
    assert w4.w4a16_sparse24_packed_bytes(0, 16) == 0
    r = lib.w4a16_sparse24_repack
    assert r(None, P_MASK, P_B, 256, 64, None) == ERR_NULL
    assert r(P_A, None, P_B, 256, 64, None) == ERR_NULL
    assert r(P_A, P_MASK, None, 256, 64, None) == ERR_NULL
    assert r(P_A, P_MASK, P_B, 200, 64, None) == ERR_SHAPE
    assert r(P_A, P_MASK, P_B, 256, 8, None) == ERR_SHAPE
    assert r(P_A, P_MASK + 4, P_B, 256, 64, None) == ERR_ALIGN
    # the packed words overlapping the codes or the mask
    assert r(P_A, P_MASK, P_A + 16, 256, 64, None) == ERR_SHAPE
    assert r(P_A, P_MASK, P_MASK + 4096 - 16, 256, 64, None) == ERR_SHAPE
    g = lib.w4a16_sparse24_gemm
    assert g(P_A, P_B, P_S, P_C, 4, 100, 64, 128, None, None) == ERR_SHAPE
    assert g(P_A, P_B, P_S, P_C, 4, 256, 64, 96, None, None) == ERR_GROUP
    assert g(None, P_B, P_S, P_C, 4, 256, 64, 128, None, None) == ERR_NULL
    assert g(P_A, P_B, P_S, P_C + 2, 4, 256, 64, 128, None, None) == ERR_ALIGN
    # C overlapping the packed 2:4 codes (K * N * 3 / 8 bytes)
    assert g(P_A, P_B, P_S, P_B + 256 * 64 * 3 // 8 - 64, 4, 256, 64, 128, None,
             None) == ERR_SHAPE
    assert g(None, None, None, None, 0, 256, 64, 128, None, None) == OK
    d = lib.w4a16_sparse24_dequant_debug
    assert d(None, P_S, P_W, 256, 64, 128, None) == ERR_NULL
    assert d(P_B, P_S, P_W, 256, 64, 96, None) == ERR_GROUP
    assert d(P_B, P_S + 2, P_W, 256, 64, 128, None) == ERR_ALIGN
    assert lib.w4a16_sparse24_workspace_bytes(4, 100, 64, 128) == 0
    buf = ctypes.create_string_buffer(64)
    assert lib.w4a16_sparse24_describe(4, 100, 64, 128, buf, 64) == ERR_SHAPE
    assert lib.w4a16_sparse24_describe(4, 256, 64, 128, None, 64) == ERR_NULL


def test_repack_and_dequant_reject_bad_arguments(lib):
    assert lib.w4a16_repack(None, P_B, 256, 64, None) == ERR_NULL
    assert lib.w4a16_repack(P_A, P_B, 200, 64, None) == ERR_SHAPE
    assert lib.w4a16_repack(P_A, P_B, 256, 8, None) == ERR_SHAPE
    assert lib.w4a16_repack(P_A + 4, P_B, 256, 64, None) == ERR_ALIGN
    assert lib.w4a16_repack(P_A, P_A + 16, 256, 64, None) == ERR_SHAPE   # overlap
    assert lib.w4a16_dequant_debug(None, P_S, P_W, 256, 64, 128, None) == ERR_NULL
    assert lib.w4a16_dequant_debug(P_B, P_S, P_W, 256, 64, 96, None) == ERR_GROUP
    assert lib.w4a16_dequant_debug(P_B, P_S, P_W, 256, 0, 128, None) == ERR_SHAPE
    assert lib.w4a16_dequant_debug(P_B, P_S + 2, P_W, 256, 64, 128, None) == ERR_ALIGN


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setenv("W4A16_LIBRARY", str(tmp_path / "missing.so"))
    mod = importlib.reload(w4)
    try:
        with pytest.raises(w4.LibraryNotBuilt):
            mod.load()
    finally:
        monkeypatch.delenv("W4A16_LIBRARY")
        importlib.reload(w4)


def test_roofline_accounting():
    # configs: 4096 x 4096, group 128, M = 16 moves 8.91 MB
    assert roofline.algorithmic_bytes(16, 4096, 4096, 128) == 8388608 + 262144 + 131072 + 131072
    assert roofline.flops(16, 4096, 4096) == 2 * 16 * 4096 * 4096
    assert roofline.bound(16, 4096, 4096, 128) == "hbm"
    assert roofline.bound(1024, 8192, 28672, 128) == "mfma"
    # the ridge between the two peaks sits near M = 80 for weight-dominated shapes
    assert roofline.bound(64, 18432, 73728, 128) == "hbm"
    assert roofline.bound(128, 18432, 73728, 128) == "mfma"


def test_forced_plan_setter(lib):
    """The tuning override parses its text and can be cleared; the launch
    path never reads the environment."""
    assert lib.w4a16_set_forced_plan(b"1,2,4,1") == OK
    assert lib.w4a16_set_forced_plan(b"1,2,4,1,2,0,0,1") == OK
    assert lib.w4a16_set_forced_plan(b"4,1,8,2,3,2") == OK
    assert lib.w4a16_set_forced_plan(b"2,4,8,0,3,4") == OK      # stream-K, eight waves
    assert lib.w4a16_set_forced_plan(b"0,0,0,0,0,-1") == OK     # the plan without stream-K
    assert lib.w4a16_set_forced_plan(b"1,2") == ERR_SHAPE        # fewer than four fields
    assert lib.w4a16_set_forced_plan(b"1,2,4,1,2,1") == ERR_SHAPE  # no tile kernel 1
    assert lib.w4a16_set_forced_plan(b"4,1,8,1,3,3") == ERR_SHAPE  # nor 3 (removed)
    assert lib.w4a16_set_forced_plan(b"x") == ERR_SHAPE
    assert lib.w4a16_set_forced_plan(None) == OK
    assert lib.w4a16_set_forced_plan(b"") == OK
    w4.w4a16_set_forced_plan("4,1,8,2,3,2")
    w4.w4a16_set_forced_plan(None)
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_set_forced_plan("1,2")
