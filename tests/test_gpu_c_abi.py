"""The library used from plain C: tests/host/c_abi_gemm.c, built with gcc
against include/patch.h, libpatch.so and the HIP runtime's C API (no C++, no
Python binding, no torch in that process), packs W with its keep mask, runs the
GEMM into bf16 and fp32 outputs and exports the packed arrays.  Its outputs are
checked here against the oracle: the exported arrays bit for bit, Y within the
oracle's tolerance, and the bf16 Y equal to the fp32 Y rounded to nearest even.

The compile-and-link check runs without a GPU; the run itself is marked gpu.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
import synthetic as I
from conftest import ROOT

LIBDIR = os.path.join(ROOT, "sparse_gemm_patch_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_program(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    if not os.path.exists(os.path.join(LIBDIR, "libpatch.so")):
        pytest.skip("libpatch.so not built")
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("no HIP headers")
    exe = tmp_path / "c_abi_gemm"
    subprocess.run([cc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "host", "c_abi_gemm.c"),
                    "-L", LIBDIR, "-lpatch", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(exe)],
                   check=True)
    return exe


def test_c_program_compiles_and_links(tmp_path):
    exe = build_c_program(tmp_path)
    # no arguments: prints its usage and exits before any HIP call
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def write_input(path, prob):
    with open(path, "wb") as f:
        f.write(np.array([prob.n, prob.k, prob.m, prob.tn, prob.tk], dtype=np.int64).tobytes())
        f.write(np.ascontiguousarray(prob.w, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(prob.bits, dtype=np.uint8).tobytes())
        f.write(np.ascontiguousarray(prob.x, dtype=np.uint16).tobytes())


def read_output(path, prob):
    raw = open(path, "rb").read()
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    n_dense, n_sparse = (int(v) for v in take(np.int64, 2))
    tiles = (prob.n // prob.tn) * (prob.k // prob.tk)
    tt = prob.tn * prob.tk
    out = {"n_dense": n_dense, "n_sparse": n_sparse,
           "y16": take(np.uint16, prob.m * prob.n).reshape(prob.m, prob.n),
           "y32": take(np.float32, prob.m * prob.n).reshape(prob.m, prob.n),
           "tile_map": take(np.uint8, tiles), "tile_slot": take(np.int32, tiles),
           "dense_vals": take(np.uint16, n_dense * tt), "sparse_vals": take(np.uint16, n_sparse * tt // 2),
           "sparse_meta": take(np.uint8, n_sparse * tt // 8)}
    assert off == len(raw)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("m,n,k,tn,tk,frac", [
    (16, 384, 512, 128, 128, 0.6),    # streaming kernel
    (300, 384, 512, 64, 128, 0.6),    # tiled kernel, ragged last row block
    (1, 256, 256, 64, 64, 1.0),       # every tile 2:4
    (40, 256, 384, 128, 64, 0.0),     # every tile dense
])
def test_c_program_against_oracle(tmp_path, m, n, k, tn, tk, frac):
    exe = build_c_program(tmp_path)
    prob = I.make_problem("c_abi", m, n, k, tn, tk, frac=frac, cfg=81)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    write_input(fin, prob)
    print(f"c_abi_gemm m={m} n={n} k={k} tile={tn}x{tk} frac={frac}", flush=True)
    r = subprocess.run([str(exe), str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = read_output(fout, prob)
    ref = O.compress(prob.w, prob.mask, tn, tk)
    assert got["n_sparse"] == int(prob.tile_sparse.sum())
    assert got["n_dense"] == prob.tile_sparse.size - got["n_sparse"]
    for key in ("tile_map", "tile_slot", "dense_vals", "sparse_vals", "sparse_meta"):
        assert np.array_equal(got[key], np.asarray(getattr(ref, key)).reshape(-1)), key
    y_ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(got["y32"].astype(np.float64), y_ref) <= O.TOL
    assert O.rel_error(I.bf16_bits_to_f32(got["y16"]).astype(np.float64), y_ref) <= O.TOL
    assert np.array_equal(got["y16"], I.f32_to_bf16_bits(got["y32"]))
