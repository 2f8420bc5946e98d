"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* tests/host/layout_roundtrip.cpp: every conversion between the exported
  row-major pools and the device's operand order, round-tripped on buffers of
  exactly the documented sizes, built with g++ -fsanitize=address,undefined.
* tests/test_abi.py again, in a child process, against a library whose host
  code is instrumented (python -m sparse_gemm_patch_amd.build --sanitize),
  with the clang ASan runtime preloaded: every argument check, the host-side
  validation of imported pools and the error paths run clean.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT


def test_layout_roundtrip_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = tmp_path / "layout_roundtrip"
    subprocess.run([cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "host", "layout_roundtrip.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "layout round trips: ok" in r.stdout


def test_abi_checks_under_sanitizers(tmp_path):
    from sparse_gemm_patch_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = B.build(sanitize=True)
    runtime = B.sanitizer_runtime()
    if not os.path.exists(runtime):
        pytest.skip("clang ASan runtime not found")
    log = tmp_path / "san"
    env = dict(os.environ, LD_PRELOAD=runtime, PATCH_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(str(log) + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-2000:] + reports)
    assert " passed" in r.stdout
