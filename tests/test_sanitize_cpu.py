"""The host side of the library (argument checks, scratch layout, the
view-length query, every reject path) under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU-only ABI tests run against a build whose
host code is instrumented (device code is built as usual)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from block_sparse_decode_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime not found")
    lib = os.path.join(B.BUILD, "sanitize", "libkvmem.so")
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + [os.path.join(ROOT, "include", "kvmem.h")]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(p) for p in srcs):
        B.build(verbose=False, sanitize=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
               LD_PRELOAD=rt, KVMEM_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
