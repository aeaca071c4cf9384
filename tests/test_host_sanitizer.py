"""Host robustness on the CPU.

* The C interface's argument checks and planner under AddressSanitizer: the
  library is rebuilt with its host code instrumented (device code as in the
  product) and tests/test_abi.py runs against it in a child process with
  the sanitizer runtime preloaded.  Any invalid host access aborts that
  process with a report.
* The workspace precondition: a workspace whose counter header is not zero
  (left over from other data) breaks the split-K hand-off, and that is the
  caller's side of a documented contract; the header must say so, and say
  that every call restores the zeros.
"""

from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import sys

import pytest

from weight_only_int4_gemm_amd import build as wbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _sources_digest() -> str:
    h = hashlib.sha256()
    for d in (wbuild.CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    h.update(" ".join(wbuild.HIPCC_FLAGS + wbuild.ASAN_HOST_FLAGS).encode())
    return h.hexdigest()


def _asan_library() -> str:
    """The instrumented library, rebuilt when a source or flag changed."""
    stamp = os.path.join(wbuild.ASAN_DIR, "sources.sha256")
    digest = _sources_digest()
    if os.path.exists(wbuild.ASAN_LIB) and os.path.exists(stamp):
        if open(stamp).read().strip() == digest:
            return wbuild.ASAN_LIB
    path = wbuild.build_host_asan()
    with open(stamp, "w") as f:
        f.write(digest + "\n")
    return path


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_abi_checks_under_address_sanitizer():
    lib = _asan_library()
    env = dict(os.environ)
    env["LD_PRELOAD"] = wbuild.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["W4A16_LIBRARY"] = lib
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_abi.py")],
                          cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=600)
    out = proc.stdout
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert re.search(r"\b\d+ passed\b", out), out[-2000:]


def test_instrumented_library_links_the_sanitizer():
    """The sanitizer build really instruments host code (guards against a
    flag that silently stops reaching the host compiler)."""
    if not os.path.exists(wbuild.ASAN_LIB):
        pytest.skip("sanitizer build not present")
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not installed")
    syms = subprocess.run([nm, "-D", wbuild.ASAN_LIB], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report" in syms or "__asan_load" in syms


def _doc_of(name: str) -> str:
    """The comment block just before a declaration in the header."""
    text = open(HEADER).read()
    i = text.index(name + "(")
    start = text.rindex("/*", 0, i)
    lines = [re.sub(r"^\s*/?\*+/?", "", ln) for ln in text[start:i].splitlines()]
    return " ".join(" ".join(lines).split())


def test_poisoned_workspace_is_a_documented_precondition():
    doc = _doc_of("size_t w4a16_workspace_bytes")
    assert "fills them with zeros once" in doc
    assert "Every call leaves the counters at zero again" in doc
    assert "header of 32-bit arrival counters" in doc
    assert "must not share a workspace" in doc
    noalloc = _doc_of("int w4a16_gemm_noalloc")
    assert "clears its counters" in noalloc
