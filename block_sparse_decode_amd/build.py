"""Build the HIP library libkvmem.so in-tree for gfx950.

    python -m block_sparse_decode_amd.build              # libkvmem.so next to this file
    python -m block_sparse_decode_amd.build --sanitize   # _build/sanitize/libkvmem.so

compiles every kernel source under csrc/ with hipcc into one shared library.
Sources are compiled in parallel, then linked.  --sanitize builds the host
code with AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
built as usual; sanitizers apply to the host side only), for running the
CPU-only ABI tests against the argument checking and scratch layout code:

    ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD=<clang's libclang_rt.asan-x86_64.so> \
        KVMEM_LIB=_build/sanitize/libkvmem.so python -m pytest tests/test_abi_cpu.py
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvmem.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: no accumulator-register reads
    # before the vector work on them (the long-chunk scorer: -16 VALU
    # instructions per 16-row operand set, 10.7 -> 10.2 ms at 10M tokens)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
SOURCES = ["kvmem_api.hip", "k_index.hip", "k_score.hip", "k_score_mfma.hip", "k_score_long.hip", "k_select.hip", "k_materialize.hip",
           "k_attend.hip", "k_append.hip",
           "k_attend_paged.hip", "k_stage.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (to LD_PRELOAD)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        import glob
        found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        p = found[-1] if found else ""
    return p


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, src.replace(".hip", ".o"))
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    out_dir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    lib = os.path.join(out_dir, "libkvmem.so") if sanitize else LIB
    extra = SANITIZE if sanitize else ()
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
