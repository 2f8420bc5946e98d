"""Build libpatch.so in-tree with hipcc for gfx950.

    python -m sparse_gemm_patch_amd.build [--sanitize]

Each HIP source is compiled to an object under ``_build/`` (in parallel), then
linked into ``sparse_gemm_patch_amd/libpatch.so``.  Packed fp32 VALU ops are
disabled for all device code.

--sanitize builds ``_build/sanitize/libpatch_sanitize.so`` instead: the same
sources with the host code (argument checks, handle management, the packed
format conversions) instrumented by AddressSanitizer and UndefinedBehavior-
Sanitizer; device code is compiled as usual.  Load it with the clang ASan
runtime preloaded (``sanitizer_runtime()``), as tests/test_host_sanitizers.py
does.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpatch.so")
SOURCES = ["api.hip", "pack.hip", "gemm.hip", "sample.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libpatch.so")
    return exe


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")


# Host-only sanitizer flags: each -fsanitize applies to the host compilation only.
SANITIZE_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_LIB = os.path.join(BUILD, "sanitize", "libpatch_sanitize.so")


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized library links against."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "/opt/rocm/lib/llvm/bin/clang"
    r = subprocess.run([clang, "--print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    out_dir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    lib = SANITIZE_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    extra = SANITIZE_FLAGS if sanitize else []
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-shared-libsan"] if sanitize else []
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
