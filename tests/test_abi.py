"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/patch.h, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import numpy as np

import pytest

from conftest import ROOT
from sparse_gemm_patch_amd import api

HEADER = os.path.join(ROOT, "include", "patch.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(patch_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.lib_path()):
        pytest.skip("libpatch.so not built")
    return api.load()


def test_header_declares_the_boundary():
    assert _declared() == sorted(api.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("cls,cname", [(api.PatchInfo, "patch_info"), (api.GemmItem, "patch_gemm_item"),
                                       (api.WeightStorage, "patch_weight_storage")])
def test_struct_layout_matches_header(tmp_path, cls, cname):
    """ctypes' structs must match what a C compiler makes of include/patch.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "patch.h"\nint main(void){\n'
                   f'  printf("%zu\\n", sizeof({cname}));\n'
                   + "".join(f'  printf("%zu\\n", offsetof({cname}, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(cls)
    assert got[1:] == [getattr(cls, f).offset for f in fields]


def _pack(lib, w=1 << 20, n=128, k=128, ldw=128, bits=1 << 20, order=0, tn=64, tk=64):
    h = ctypes.c_void_p(0xDEAD)
    info = api.PatchInfo()
    st = lib.patch_pack(ctypes.c_void_p(w), n, k, ldw, ctypes.c_void_p(bits), order, tn, tk, None,
                        ctypes.byref(h), ctypes.byref(info))
    return st, h.value


def test_pack_argument_errors(lib):
    # each of these is rejected before any HIP call, and *out is cleared
    assert _pack(lib, tn=32) == (2, None)                 # tile side not 64/128
    assert _pack(lib, tk=256) == (2, None)
    assert _pack(lib, n=100) == (2, None)                 # ragged N
    assert _pack(lib, k=96) == (2, None)                  # ragged K
    assert _pack(lib, n=-64) == (2, None)
    assert _pack(lib, order=7) == (1, None)               # bad bit order
    assert _pack(lib, w=0) == (1, None)                   # NULL pointers
    assert _pack(lib, bits=0) == (1, None)
    assert _pack(lib, w=(1 << 20) + 2) == (1, None)       # misaligned
    assert _pack(lib, ldw=120) == (1, None)               # ldw < k
    assert _pack(lib, ldw=132) == (1, None)               # ldw not a multiple of 8
    st = lib.patch_pack(None, 0, 0, 0, None, 0, 64, 64, None, None, None)
    assert st == 1                                        # out == NULL


@pytest.mark.parametrize("n,k", [(1 << 40, 1 << 40), (1 << 62, 128), (128, 1 << 62), (46400, 46336)])
def test_pack_rejects_shapes_past_the_weight_limit(lib, n, k):
    """Shapes whose weight count exceeds 2^31 - 1, including ones where N * K itself would
    overflow 64 bits, are rejected as PATCH_E_SHAPE before any HIP call."""
    assert _pack(lib, n=n, k=k, ldw=k) == (2, None)
    assert b"2^31" in lib.patch_last_error()


def test_error_text_names_the_problem(lib):
    _pack(lib, tn=32)
    assert b"64 or 128" in lib.patch_last_error()
    _pack(lib, n=100)
    assert b"whole number" in lib.patch_last_error()


def test_gemm_and_unpack_argument_errors(lib):
    assert lib.patch_gemm(None, None, 1, 64, None, 64, 0, None) == 1
    assert lib.patch_gemm_kernel(None, None, 1, 64, None, 64, 0, 0, 0, None) == 1
    assert lib.patch_unpack(None, None, 64, None) == 1
    assert lib.patch_get_info(None, None) == 1
    assert lib.patch_export(None, None, None, None, None, None) == 1
    assert lib.patch_mask_unpack(None, 8, 5, None, None) == 1      # bad order
    assert lib.patch_mask_unpack(None, -1, 0, None, None) == 1     # negative count
    assert lib.patch_mask_unpack(None, 0, 0, None, None) == 0      # empty is a no-op
    lib.patch_destroy(None)                                        # NULL is a no-op


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "_LIB", None)
    monkeypatch.setenv("PATCH_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(api.PatchError):
        api.load()


def test_grouped_argument_errors(lib):
    """Rejected before any HIP call; the failing product is named."""
    items = (api.GemmItem * 17)()
    assert lib.patch_gemm_grouped(items, 0, 0, None) == 0            # empty group: no-op
    assert lib.patch_gemm_grouped(None, 0, 0, None) == 0
    assert lib.patch_gemm_grouped(None, 1, 0, None) == 1             # items NULL
    assert lib.patch_gemm_grouped(items, 17, 0, None) == 1           # more than 16
    assert b"0..16" in lib.patch_last_error()
    assert lib.patch_gemm_grouped(items, -1, 0, None) == 1
    assert lib.patch_gemm_grouped(items, 2, 9, None) == 1            # bad dtype
    assert lib.patch_gemm_grouped(items, 2, 0, None) == 1            # NULL handles
    assert lib.patch_last_error().startswith(b"product 0: weight handle is NULL")
    assert lib.patch_gemm_grouped_kernel(items, 2, 0, 7, 0, None) == 1   # bad kernel
    assert lib.patch_gemm_grouped_kernel(items, 2, 0, 1, 96, None) == 1  # bad block rows


def _import(lib, n=128, k=128, tn=64, tk=64, tile_map=None, dense=True, sparse=True, meta=None):
    tiles = (n // tn) * (k // tk) if n % tn == 0 and k % tk == 0 and tn in (64, 128) and tk in (64, 128) else 1
    tm = np.full(tiles, 1, np.uint8) if tile_map is None else np.asarray(tile_map, np.uint8)
    ns = int((tm == 1).sum())
    nd = int((tm == 0).sum())
    dv = np.zeros(max(nd * tn * tk, 1), np.uint16)
    sv = np.zeros(max(ns * tn * tk // 2, 1), np.uint16)
    sm = np.full(max(ns * tn * tk // 8, 1), 0x44, np.uint8) if meta is None else meta
    h = ctypes.c_void_p(0xBEEF)
    info = api.PatchInfo()
    st = lib.patch_import(n, k, tn, tk, tm.ctypes.data, dv.ctypes.data if dense else None,
                          sv.ctypes.data if sparse else None, sm.ctypes.data if sparse else None, None,
                          ctypes.byref(h), ctypes.byref(info))
    return st, h.value, info


def test_import_argument_errors(lib):
    """patch_import validates the exported format on the host before any HIP call."""
    assert _import(lib, tn=32)[:2] == (2, None)                     # tile side
    assert _import(lib, n=100)[:2] == (2, None)                     # ragged N
    assert _import(lib, tile_map=[0, 1, 2, 1])[:2] == (1, None)     # not a tile type
    assert b"tile_map[2]" in lib.patch_last_error()
    assert _import(lib, tile_map=[0, 1, 1, 1], dense=False)[:2] == (1, None)   # dense pool missing
    assert _import(lib, tile_map=[0, 1, 1, 1], sparse=False)[:2] == (1, None)  # 2:4 pools missing
    st = lib.patch_import(128, 128, 64, 64, None, None, None, None, None, None, None)
    assert st == 1                                                  # out == NULL


@pytest.mark.parametrize("code", [0, 1, 2, 3, 5, 6, 7, 10, 11, 15])
def test_import_rejects_illegal_codes(lib, code):
    """Only the six codes i0 | i1 << 2 with i0 < i1 are legal; the first bad one is located."""
    tm = np.array([0, 1, 0, 1], np.uint8)          # 64x64 tiles: slot 1 of the 2:4 pool is tile 3
    meta = np.full(2 * 64 * 64 // 8, 0x44, np.uint8)
    row, group = 17, 9                              # group 9 is the high nibble of byte 4 of the row
    meta[64 * 64 // 8 + row * 8 + group // 2] = (code << 4) | 0x4
    st, h, info = _import(lib, tile_map=tm, meta=meta)
    assert (st, h) == (3, None)
    assert (info.bad_tile, info.bad_row, info.bad_group) == (3, row, group)


def test_sample_mask_argument_errors(lib):
    f = ctypes.c_void_p(1 << 20)
    assert lib.patch_sample_mask(f, None, f, None, 128, 128, 64, 64, 25.0, 7, f, None) == 1   # bad order
    assert lib.patch_sample_mask(f, None, f, None, 128, 128, 64, 32, 25.0, 0, f, None) == 2   # tile side
    assert lib.patch_sample_mask(f, None, f, None, 100, 128, 64, 64, 25.0, 0, f, None) == 2   # ragged N
    assert lib.patch_sample_mask(None, None, f, None, 128, 128, 64, 64, 25.0, 0, f, None) == 1
    assert lib.patch_sample_mask(f, None, f, None, 128, 128, 64, 64, 25.0, 0, None, None) == 1
    g = ctypes.c_void_p((1 << 20) + 2)
    assert lib.patch_sample_mask(f, g, f, None, 128, 128, 64, 64, 25.0, 0, f, None) == 1      # misaligned
    assert lib.patch_sample_mask(None, None, None, None, 0, 128, 64, 64, 25.0, 0, None, None) == 0  # empty


def test_header_max_ldx():
    text = open(HEADER).read()
    assert re.search(r"#define PATCH_MAX_LDX 4194304LL", text)


def test_pack_noalloc_argument_errors(lib):
    """Rejected before any HIP call; *out is cleared."""
    st = api.WeightStorage()
    h = ctypes.c_void_p(0xDEAD)
    vp = ctypes.c_void_p

    def call(n=128, k=128, tn=64, tk=64, order=0, storage=True, out=True, w=1 << 20):
        h.value = 0xDEAD
        return lib.patch_pack_noalloc(vp(w), n, k, k, vp(1 << 20), order, tn, tk, None, vp(1 << 20), vp(1 << 20),
                                      vp(1 << 20), 1 << 16, vp(1 << 20), 1 << 16, vp(1 << 20), 1 << 16,
                                      ctypes.byref(st) if storage else None, ctypes.byref(h) if out else None, None)
    assert call(out=False) == 1
    assert call(storage=False) == 1 and h.value is None
    assert call(order=3) == 1 and h.value is None
    assert call(tn=32) == 2 and h.value is None
    assert call(n=100) == 2
    # more than PATCH_MAX_WEIGHTS (2^31 - 1) weights: the pools' 32-bit offsets would wrap
    assert call(n=65536, k=32768) == 2 and h.value is None
    assert b"2^31" in lib.patch_last_error()
    assert call(w=0) == 1
    assert call(w=(1 << 20) + 2) == 1


def test_workspace_argument_errors(lib):
    """Rejected before any HIP call."""
    vp = ctypes.c_void_p
    n = ctypes.c_int64(-1)
    assert lib.patch_gemm_workspace_size(None, 16, ctypes.byref(n)) == 1                 # NULL handle
    assert lib.patch_gemm_workspace_size(vp(1 << 20), 16, None) == 1                     # NULL result
    assert lib.patch_gemm_workspace_size(vp(1 << 20), -1, ctypes.byref(n)) == 1          # m < 0
    assert lib.patch_gemm_with_workspace(None, None, 1, 64, None, 64, 0, None, 0, None) == 1
    assert lib.patch_gemm_with_workspace(vp(1 << 20), vp(1 << 20), 1, 64, vp(1 << 20), 64, 0,
                                         vp((1 << 20) + 4), 1 << 16, None) == 1           # misaligned workspace
    assert b"16-byte" in lib.patch_last_error()
    assert lib.patch_gemm_with_workspace(vp(1 << 20), vp(1 << 20), 1, 64, vp(1 << 20), 64, 0,
                                         vp(1 << 20), -8, None) == 1                      # negative size
