"""Build libw4a16.so from the HIP sources in ``csrc/`` for gfx950.

    python -m weight_only_int4_gemm_amd.build

Compiles each translation unit with hipcc (in parallel) into ``_build/`` at
the repository root and links ``weight_only_int4_gemm_amd/libw4a16.so``, then
the measurement probes (``csrc/probes.hip``) into ``libw4a16_probes.so``.
Cross-compiles without a GPU.  Always rebuilds.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
PROBES_LIB = os.path.join(PKG, "libw4a16_probes.so")
SOURCES = ["api.hip", "gemm.hip", "gemm_lds.hip", "gemm_sk.hip", "gemm_sk_fmt.hip", "repack.hip", "dequant.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep the kernels' per-lane arrays (register slots, pointers) out of LDS;
    # once the loops are unrolled they are plain registers
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = min(len(cmds), int(os.environ.get("MAX_JOBS", "8")) or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the measurement probes: a library of their own, loaded by bench.py only
    pobj = os.path.join(BUILD, "probes.o")
    _run([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, "probes.hip"), "-o", pobj])
    tmp = PROBES_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, pobj])
    os.replace(tmp, PROBES_LIB)
    return LIB


# Host-side AddressSanitizer build: the same sources and device code, with
# the host half of every file instrumented.  It is a test build for the
# argument checks and planner (tests/test_host_sanitizer.py loads it into a
# process with the sanitizer runtime preloaded); kernels are never launched
# from it.
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libw4a16_asan.so")
ASAN_HOST_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer "
                   "-Xarch_host -g").split()


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that matches hipcc, for LD_PRELOAD."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return hits[-1]


def build_host_asan() -> str:
    hipcc = _hipcc()
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *ASAN_HOST_FLAGS, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    jobs = min(len(cmds), int(os.environ.get("MAX_JOBS", "8")) or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = ASAN_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_HOST_FLAGS[:2], "-o", tmp,
          *objs])
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
