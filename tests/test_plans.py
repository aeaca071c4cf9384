"""The plan heuristic on the CPU (w4a16_plan_describe takes the compute-unit
count as an argument, so no device is needed): which kernel each batch and
layer size gets, and that every compiled kernel instantiation is one some
plan picks (none is dead weight in the library)."""

from __future__ import annotations

import os
import re

import pytest

import weight_only_int4_gemm_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_int4_gemm_amd", "csrc")
CUS = 256  # MI355X

F16, F16ZP, BF16, BF16ZP, W8, SP24 = range(6)


def plan(M, K, N, fmt=F16, group=128):
    return w4.w4a16_plan_describe(M, K, N, group, fmt, CUS)


def test_stream_k_takes_9_to_128_rows_on_large_layers():
    K, N = 18432, 73728
    for M, name in ((9, "1,4,4,8"), (16, "1,4,4,8"), (17, "2,4,3,8"), (32, "2,4,3,8"),
                    (33, "4,4,3,8"), (64, "4,4,3,8")):
        for fmt in (F16, F16ZP, BF16, BF16ZP):
            assert plan(M, K, N, fmt).startswith(f"gemm_sk_kernel<{name}>"), (M, fmt)
        assert not plan(M, K, N, W8).startswith("gemm_sk_kernel<"), M
        assert not plan(M, K, N, SP24).startswith("gemm_sk_kernel<"), M
    for M in (65, 96, 128):
        for fmt in (F16, F16ZP, BF16, BF16ZP):
            assert plan(M, K, N, fmt).startswith("gemm_sk_kernel<8,2,3,8>"), (M, fmt)
    assert plan(128, 28672, 8192).startswith("gemm_sk_kernel<8,2,3,8>")
    for M in (1, 8, 129, 1024):
        assert not plan(M, K, N).startswith("gemm_sk_kernel<"), M
    for K2, N2 in ((4096, 4096), (4096, 12288), (4096, 22016), (11008, 4096), (8192, 28672),
                   (28672, 8192), (13824, 5120)):
        for M in (16, 32, 64):
            assert not plan(M, K2, N2).startswith("gemm_sk_kernel<"), (M, K2, N2)
    for K2, N2 in ((4096, 4096), (4096, 12288), (4096, 22016), (11008, 4096), (8192, 28672),
                   (13824, 5120)):
        assert not plan(128, K2, N2).startswith("gemm_sk_kernel<"), (K2, N2)
    for M in (512, 1024, 4096):
        assert not plan(M, 8192, 28672).startswith("gemm_sk_kernel<"), M


def test_narrow_layers_17_to_32_rows_take_64_row_tiles():
    """17 to 32 rows on narrow layers (at most cus/8 column tiles of 256,
    4096 <= K <= 8192, dense codes): 64 x 128 tiles; wider layers, deeper K,
    2:4 codes and 16 rows keep the 32 x 256 (16 x 256) tiles."""
    for M in (17, 24, 32):
        for K, N in ((4096, 4096), (4096, 6144), (4096, 8192), (5120, 5120), (8192, 4096)):
            for fmt in (F16, F16ZP, BF16, BF16ZP, W8):
                assert plan(M, K, N, fmt).startswith("gemm_lds_kernel<4,1,1,8,3>"), (M, K, N, fmt)
        for K, N in ((4096, 12288), (4096, 22016), (11008, 4096), (13824, 5120), (2048, 4096)):
            assert plan(M, K, N).startswith("gemm_lds_kernel<2,2,1,8,4>"), (M, K, N)
        assert not plan(M, 4096, 4096, SP24).startswith("gemm_lds_kernel<4,1,1,8,3>"), M
    assert plan(16, 4096, 8192).startswith("gemm_lds_kernel<1,2,1,8,4>")


def test_few_tiles_keep_eight_k_blocks_per_split():
    """With fewer tiles than compute units the LDS kernel splits K, but from
    K = 4096 on into ranges of at least eight K blocks (deep K keeps the cap
    of eight splits; below K = 4096 the old cap of K/512)."""
    def splits(d):
        return int(re.search(r"splits=(\d+)", d).group(1))
    assert splits(plan(32, 4096, 4096)) == 4          # 32 tiles: 8 wanted, 32/8 allowed
    assert splits(plan(48, 4096, 4096)) == 4
    assert splits(plan(16, 4096, 8192)) == 4
    assert splits(plan(16, 6144, 8192)) == 6
    assert splits(plan(32, 11008, 4096)) == 8         # deep enough: eight
    assert splits(plan(32, 28672, 8192)) == 8
    assert splits(plan(16, 2048, 8192)) == 4          # below K = 4096: K/512
    for M, K, N in ((32, 4096, 4096), (16, 4096, 8192), (16, 6144, 8192), (48, 5120, 5120)):
        d = plan(M, K, N)
        assert (K // 128) // splits(d) >= 8, (M, K, N, d)


def test_activations_in_lds_rule():
    """The streaming kernel stages its activations in LDS exactly when the
    batch has at most four rows, those rows over a workgroup's K range fit in
    32 KiB, and the activations are FP16 (formats 0, 1 and 4)."""
    staged = "activations=lds"
    for fmt in (F16, F16ZP, W8):
        assert staged in plan(1, 4096, 12288, fmt)
        assert staged in plan(4, 4096, 4096, fmt)           # 4 x 4096 x 2 = 32 KiB
        assert staged not in plan(4, 4224, 4096, fmt)       # 33 KiB
        assert staged not in plan(5, 4096, 4096, fmt)
        assert staged in plan(2, 16384, 64, fmt)            # split K: 43 blocks per range
    for fmt in (BF16, BF16ZP, SP24):
        for M in (1, 2, 4):
            assert staged not in plan(M, 4096, 12288, fmt), (M, fmt)
    assert staged not in plan(1, 18432, 73728)              # 36 KiB per row
    for M in (16, 128, 1024):                               # other kernels never
        assert staged not in plan(M, 4096, 4096), M


def test_lds_tail_split():
    """More tiles than compute units and a last wave at most half full:
    whole waves' tiles run whole, the rest are split in two along K."""
    d = plan(1024, 8192, 28672)   # 8 x 112 = 896 tiles: 768 whole + 128 split 2 ways
    assert d.startswith("gemm_lds_kernel<8,2,1,8,3>") and "whole=768 splits=2 " in d, d
    assert "grid=1024x1x1" in d, d
    d = plan(512, 8192, 28672)    # 448 tiles: the last wave three-quarters full, nothing split
    assert "splits=1 " in d and "workspace=0" in d, d
    d = plan(4096, 8192, 28672)   # 3584 tiles: 14 full waves, nothing split
    assert "splits=1 " in d and "workspace=0" in d, d
    w4.w4a16_set_forced_plan("8,2,8,1,3,2")   # a forced plan is taken as it is
    try:
        assert "splits=1 " in plan(1024, 8192, 28672)
    finally:
        w4.w4a16_set_forced_plan(None)


def test_plan_describe_checks_its_arguments():
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4096, 4096, 128, 6, CUS)    # no such format
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4096, 4096, 128, F16, 0)    # no compute units
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_plan_describe(16, 4000, 4096, 128, F16, CUS)  # K not a multiple of 128


def _macro_tuples(path, name):
    """The X(...) argument tuples of a variant-list macro (following one
    level of macros it includes)."""
    src = open(path).read()
    m = re.search(r"#define " + name + r"\(X\)(.*?)(?:\n\n|\n(?=[^ \\]))", src, re.S)
    assert m, name
    body = m.group(1)
    out = [tuple(int(x) for x in t.split(",")) for t in re.findall(r"X\(([\d, ]+)\)", body)]
    for inner in re.findall(r"(W4A16_\w+_VARIANTS)\(X\)", body):
        out += _macro_tuples(path, inner)
    return out


def compiled_variants():
    """{(kernel, format): [template tuple as w4a16_describe prints it]}."""
    g, l, k = (os.path.join(CSRC, f) for f in ("gemm.hip", "gemm_lds.hip", "gemm_sk.hpp"))
    out = {}
    for fmt in (F16, F16ZP, BF16, BF16ZP, W8):
        for t in _macro_tuples(g, "W4A16_VARIANTS"):
            out.setdefault(("gemm_kernel", fmt), set()).add(t)
    for fmt in (BF16, BF16ZP, W8):
        for t in _macro_tuples(g, "W4A16_SCALED_WEIGHT_VARIANTS"):
            out.setdefault(("gemm_kernel", fmt), set()).add(t)
    for t in _macro_tuples(g, "W4A16_SP_VARIANTS"):
        out.setdefault(("gemm_kernel", SP24), set()).add(t)
    for fmt in (F16, F16ZP, BF16, BF16ZP, W8):
        for t in _macro_tuples(l, "W4A16_LDS_VARIANTS"):
            out.setdefault(("gemm_lds_kernel", fmt), set()).add(t)
    for t in _macro_tuples(l, "W4A16_LDS_SP_VARIANTS"):
        out.setdefault(("gemm_lds_kernel", SP24), set()).add(t)
    for fmt in (F16, F16ZP, BF16, BF16ZP):
        for t in _macro_tuples(k, "W4A16_SK_VARIANTS"):
            # printed as <mb,nb,depth,wn>, the macro's own order
            out.setdefault(("gemm_sk_kernel", fmt), set()).add(t)
    return out


MS = [1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 24, 32, 33, 48, 64, 65, 96, 128, 129, 192, 256, 512,
      1024, 2048, 4096]
KS = [128, 256, 512, 1024, 2048, 3584, 4096, 8192, 11008, 13824, 18432, 28672]
NS = [16, 64, 208, 512, 1024, 2048, 4096, 5120, 8192, 12288, 14336, 22016, 28672, 36864,
      65536, 73728]


def reachable_variants():
    seen = {}
    for fmt in range(6):
        for M in MS:
            for K in KS:
                for N in NS:
                    for group in ((128, K) if fmt != SP24 else (128,)):
                        d = plan(M, K, N, fmt, group)
                        name, args = re.match(r"(\w+)<([\d,]+)>", d).groups()
                        seen.setdefault((name, fmt), set()).add(
                            tuple(int(x) for x in args.split(",")))
    return seen


def test_every_compiled_variant_is_one_a_plan_picks():
    compiled = compiled_variants()
    seen = reachable_variants()
    dead = {key: sorted(v - seen.get(key, set())) for key, v in compiled.items()}
    dead = {k: v for k, v in dead.items() if v}
    assert not dead, f"compiled but never planned: {dead}"
    missing = {key: sorted(v - compiled.get(key, set())) for key, v in seen.items()}
    missing = {k: v for k, v in missing.items() if v}
    assert not missing, f"planned but not compiled: {missing}"


def test_five_to_eight_rows_stream_on_wide_layers_in_fp16():
    """FP16 formats at M = 5..8 on layers with N >= 8192: the streaming
    kernel, unsplit, 64-column tiles of four waves from 1536 column blocks
    and 32-column tiles of eight waves below; the other formats keep the
    LDS kernel there."""
    for K, N, name in ((8192, 28672, "1,4,4,2"), (4096, 22016, "1,2,8,2"),
                       (4096, 12288, "1,2,8,2"), (28672, 8192, "1,2,8,2"),
                       (18432, 73728, "1,4,4,2")):
        for M in (5, 8):
            for fmt in (F16, F16ZP):
                d = plan(M, K, N, fmt)
                assert d.startswith(f"gemm_kernel<{name}>") and " splits=1 " in d, (K, N, M, d)
        for fmt in (BF16, W8):
            d = plan(8, K, N, fmt)
            assert d.startswith("gemm_kernel<1,4,4,2>" if N == 73728 else "gemm_lds_kernel<"), d
    # unchanged: four rows and fewer, nine rows and more, narrow layers
    assert plan(4, 28672, 8192).startswith("gemm_kernel<1,2,8,2>") and " splits=3 " in plan(4, 28672, 8192)
    assert plan(9, 4096, 12288).startswith("gemm_lds_kernel<")
    assert plan(8, 13824, 5120).startswith("gemm_kernel<1,4,4,2>") and " splits=8 " in plan(8, 13824, 5120)
