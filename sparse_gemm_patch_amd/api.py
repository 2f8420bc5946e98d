"""ctypes binding over libpatch.so (include/patch.h).

Argument marshalling only: every step of packing, unpacking and the GEMM runs
in the library's HIP kernels.  PyTorch supplies device memory and the current
stream.  If the library is missing, every call raises PatchError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))

STATUS = {0: "PATCH_OK", 1: "PATCH_E_INVALID_ARG", 2: "PATCH_E_SHAPE", 3: "PATCH_E_MASK", 4: "PATCH_E_HIP",
          5: "PATCH_E_NOMEM", 6: "PATCH_E_UNSUPPORTED"}
BIT_ORDER = {"big": 0, "msb": 0, "little": 1, "lsb": 1}
KERNEL = {"auto": 0, "tiled": 1, "stream": 2}
OUT_DTYPE = {torch.bfloat16: 0, torch.float32: 1}
DENSE, SPARSE24 = 0, 1

# Exported entry points; kept in step with include/patch.h.
SYMBOLS = ("patch_pack", "patch_gemm", "patch_gemm_kernel", "patch_gemm_grouped", "patch_gemm_grouped_kernel",
           "patch_gemm_with_workspace", "patch_gemm_workspace_size", "patch_unpack", "patch_mask_unpack", "patch_get_info", "patch_export", "patch_import",
           "patch_sample_mask", "patch_pack_noalloc", "patch_destroy", "patch_last_error")
MAX_GROUP = 16


class PatchInfo(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("tiles_n", ctypes.c_int64), ("tiles_k", ctypes.c_int64),
                ("n_dense", ctypes.c_int64), ("n_sparse", ctypes.c_int64), ("bytes_dense", ctypes.c_int64),
                ("bytes_sparse_vals", ctypes.c_int64), ("bytes_sparse_meta", ctypes.c_int64),
                ("sparsity", ctypes.c_double), ("bad_tile", ctypes.c_int64), ("bad_row", ctypes.c_int64),
                ("bad_group", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class WeightStorage(ctypes.Structure):
    """Host storage of a handle made by patch_pack_noalloc (patch_weight_storage)."""
    _fields_ = [("words", ctypes.c_uint64 * 64)]


class GemmItem(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("m", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class PatchError(RuntimeError):
    def __init__(self, status: int, message: str, info: Optional[dict] = None):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        self.info = info


_LIB = None


def lib_path() -> str:
    return os.environ.get("PATCH_LIB", os.path.join(HERE, "libpatch.so"))


def load() -> ctypes.CDLL:
    """Load libpatch.so and declare the C signatures (raises PatchError if absent)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise PatchError(-1, f"{path} is not built (run python -m sparse_gemm_patch_amd.build)")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.patch_pack.argtypes = [vp, i64, i64, i64, vp, ctypes.c_int, i32, i32, vp, ctypes.POINTER(vp),
                             ctypes.POINTER(PatchInfo)]
    L.patch_gemm.argtypes = [vp, vp, i64, i64, vp, i64, ctypes.c_int, vp]
    L.patch_gemm_kernel.argtypes = [vp, vp, i64, i64, vp, i64, ctypes.c_int, ctypes.c_int, i32, vp]
    L.patch_gemm_grouped.argtypes = [ctypes.POINTER(GemmItem), i32, ctypes.c_int, vp]
    L.patch_gemm_with_workspace.argtypes = [vp, vp, i64, i64, vp, i64, ctypes.c_int, vp, i64, vp]
    L.patch_gemm_workspace_size.argtypes = [vp, i64, ctypes.POINTER(i64)]
    L.patch_gemm_grouped_kernel.argtypes = [ctypes.POINTER(GemmItem), i32, ctypes.c_int, ctypes.c_int, i32, vp]
    L.patch_unpack.argtypes = [vp, vp, i64, vp]
    L.patch_mask_unpack.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    L.patch_get_info.argtypes = [vp, ctypes.POINTER(PatchInfo)]
    L.patch_export.argtypes = [vp, vp, vp, vp, vp, vp]
    L.patch_import.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(PatchInfo)]
    L.patch_sample_mask.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, ctypes.c_float, ctypes.c_int, vp, vp]
    L.patch_pack_noalloc.argtypes = [vp, i64, i64, i64, vp, ctypes.c_int, i32, i32, vp, vp, vp, vp, i64, vp, i64, vp,
                                     i64, vp, ctypes.POINTER(vp), ctypes.POINTER(PatchInfo)]
    L.patch_destroy.argtypes = [vp]
    L.patch_destroy.restype = None
    L.patch_last_error.argtypes = []
    L.patch_last_error.restype = ctypes.c_char_p
    for name in ("patch_pack", "patch_gemm", "patch_gemm_kernel", "patch_gemm_grouped", "patch_gemm_grouped_kernel",
                 "patch_gemm_with_workspace", "patch_gemm_workspace_size", "patch_unpack", "patch_mask_unpack", "patch_get_info", "patch_export", "patch_import",
                 "patch_sample_mask", "patch_pack_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def _raise(st: int, info: Optional[dict] = None):
    msg = load().patch_last_error().decode(errors="replace")
    raise PatchError(st, msg, info)


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_cuda(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _row_major_2d(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along its last dimension")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


class PackedWeight:
    """A packed hybrid dense / 2:4 weight (owns the library handle)."""

    def __init__(self, handle: ctypes.c_void_p, info: dict, device: torch.device):
        self._h = handle
        self.info = info
        self.device = device
        self.n, self.k = info["n"], info["k"]

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _LIB is not None:
            _LIB.patch_destroy(h)

    def _operands(self, x: torch.Tensor, out: Optional[torch.Tensor], out_dtype: torch.dtype):
        """Checks X, allocates or checks Y; returns (m, ldx, out, ldy)."""
        _check_cuda(x, "x", torch.bfloat16)
        ldx = _row_major_2d(x, "x")
        if x.shape[1] != self.k:
            raise ValueError(f"x has {x.shape[1]} columns, weight has k = {self.k}")
        if out_dtype not in OUT_DTYPE:
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        m = x.shape[0]
        if out is None:
            ldy = (self.n + 7) // 8 * 8
            buf = torch.empty((m, ldy), dtype=out_dtype, device=x.device)
            out = buf[:, :self.n]
        else:
            _check_cuda(out, "out", out_dtype)
            if tuple(out.shape) != (m, self.n):
                raise ValueError(f"out must be [{m}][{self.n}]")
        return m, ldx, out, _row_major_2d(out, "out")

    def workspace_size(self, m: int) -> int:
        """Bytes of workspace with which gemm(..., workspace=...) splits K for m rows (0: no split)."""
        n = ctypes.c_int64(0)
        st = load().patch_gemm_workspace_size(self._h, int(m), ctypes.byref(n))
        if st:
            _raise(st)
        return n.value

    def gemm(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
             kernel: str = "auto", block_m: int = 0, stream=None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Y = X . W_masked^T for X bf16 [m][k]; returns Y [m][n] (bf16 or fp32).

        kernel "tiled" takes block_m (X rows per workgroup: 256, 192, 128 or 64; 0 =
        the library's choice).  A workspace (a device tensor, kernel "auto" only) goes
        to patch_gemm_with_workspace, which splits K when it holds workspace_size(m)
        bytes."""
        m, ldx, out, ldy = self._operands(x, out, out_dtype)
        if workspace is not None:
            if kernel != "auto":
                raise ValueError("a workspace is taken with kernel='auto' only")
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous device tensor")
            st = load().patch_gemm_with_workspace(self._h, ctypes.c_void_p(x.data_ptr()), m, ldx,
                                                  ctypes.c_void_p(out.data_ptr()), ldy, OUT_DTYPE[out_dtype],
                                                  ctypes.c_void_p(workspace.data_ptr()),
                                                  workspace.numel() * workspace.element_size(), _stream_handle(stream))
            if st:
                _raise(st)
            return out
        st = load().patch_gemm_kernel(self._h, ctypes.c_void_p(x.data_ptr()), m, ldx, ctypes.c_void_p(out.data_ptr()),
                                      ldy, OUT_DTYPE[out_dtype], KERNEL[kernel],
                                      int(block_m if kernel == "tiled" else 0),
                                      _stream_handle(stream))
        if st:
            _raise(st)
        return out

    def unpack(self, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Masked dense W (bf16 [n][k]), pruned weights +0.0."""
        if out is None:
            out = torch.empty((self.n, self.k), dtype=torch.bfloat16, device=self.device)
        # shape first: the kernel writes n rows of k values at out's row stride
        if tuple(out.shape) != (self.n, self.k):
            raise ValueError(f"out must be [{self.n}][{self.k}], got {list(out.shape)}")
        _check_cuda(out, "out", torch.bfloat16)
        ldw = _row_major_2d(out, "out") if out.numel() else self.k
        st = load().patch_unpack(self._h, ctypes.c_void_p(out.data_ptr()), ldw, _stream_handle(stream))
        if st:
            _raise(st)
        return out

    def export(self) -> dict:
        """Host copies of the packed arrays (numpy): tile_map, tile_slot, dense_vals, sparse_vals, sparse_meta."""
        i = self.info
        tn, tk = i["tile_n"], i["tile_k"]
        T = i["tiles_n"] * i["tiles_k"]
        arrs = {"tile_map": np.zeros(T, np.uint8), "tile_slot": np.zeros(T, np.int32),
                "dense_vals": np.zeros((i["n_dense"], tn, tk), np.uint16),
                "sparse_vals": np.zeros((i["n_sparse"], tn, tk // 2), np.uint16),
                "sparse_meta": np.zeros((i["n_sparse"], tn, tk // 8), np.uint8)}
        ptr = {k: (ctypes.c_void_p(v.ctypes.data) if v.size else None) for k, v in arrs.items()}
        st = load().patch_export(self._h, ptr["tile_map"], ptr["tile_slot"], ptr["dense_vals"], ptr["sparse_vals"],
                                 ptr["sparse_meta"])
        if st:
            _raise(st)
        return arrs


def gemm_grouped(products, outs=None, out_dtype: torch.dtype = torch.bfloat16, kernel: str = "auto",
                 block_m: int = 0, stream=None) -> list:
    """Several independent products in one launch per kernel.

    products: sequence of (PackedWeight, X) pairs (at most 16); outs: None or a
    matching sequence of Y tensors / None.  Returns the Y list; each Y equals
    what PackedWeight.gemm gives for its pair alone, bit for bit."""
    products = list(products)
    if len(products) > MAX_GROUP:
        raise ValueError(f"at most {MAX_GROUP} products per group, got {len(products)}")
    outs = [None] * len(products) if outs is None else list(outs)
    if len(outs) != len(products):
        raise ValueError("outs must match products")
    items = (GemmItem * max(len(products), 1))()
    for i, ((pw, x), out) in enumerate(zip(products, outs)):
        m, ldx, out, ldy = pw._operands(x, out, out_dtype)
        outs[i] = out
        items[i] = GemmItem(pw._h, x.data_ptr(), m, ldx, out.data_ptr(), ldy)
    st = load().patch_gemm_grouped_kernel(items, len(products), OUT_DTYPE[out_dtype], KERNEL[kernel],
                                          int(block_m if kernel == "tiled" else 0), _stream_handle(stream))
    if st:
        _raise(st)
    return outs


PACKED_ARRAYS = ("tile_map", "dense_vals", "sparse_vals", "sparse_meta")


def import_packed(arrays: dict, n: int, k: int, tile=(128, 128), device=None, stream=None) -> PackedWeight:
    """Rebuild a packed weight from the arrays PackedWeight.export returns (tile_slot is implied
    by tile_map and ignored).  The arrays are host numpy arrays; the weight lands on `device`."""
    tn, tk = int(tile[0]), int(tile[1])
    n, k = int(n), int(k)
    if tn not in (64, 128) or tk not in (64, 128) or n < 0 or k < 0 or n % tn or k % tk:
        raise ValueError(f"W {n}x{k} is not a whole number of {tn}x{tk} tiles (each side 64 or 128)")
    tm = np.ascontiguousarray(arrays["tile_map"], dtype=np.uint8).reshape(-1)
    # the library reads exactly (n/tn)*(k/tk) tile-map bytes and sizes the pools from them
    if tm.size != (n // tn) * (k // tk):
        raise ValueError(f"tile_map has {tm.size} entries, a {n}x{k} weight in {tn}x{tk} tiles has "
                         f"{(n // tn) * (k // tk)}")
    nd = int(np.count_nonzero(tm == DENSE))
    ns = int(np.count_nonzero(tm == SPARSE24))
    want = {"dense_vals": (np.uint16, nd * tn * tk), "sparse_vals": (np.uint16, ns * tn * tk // 2),
            "sparse_meta": (np.uint8, ns * tn * tk // 8)}
    host = {"tile_map": tm}
    for key, (dt, size) in want.items():
        a = np.ascontiguousarray(arrays[key])
        if a.dtype != dt or a.size != size:
            raise ValueError(f"{key}: expected {size} values of {np.dtype(dt).name}, got {a.size} of {a.dtype}")
        host[key] = a.reshape(-1)
    ptr = {key: (ctypes.c_void_p(a.ctypes.data) if a.size else None) for key, a in host.items()}
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    h = ctypes.c_void_p()
    info = PatchInfo()
    with torch.cuda.device(dev):
        st = load().patch_import(int(n), int(k), tn, tk, ptr["tile_map"], ptr["dense_vals"], ptr["sparse_vals"],
                                 ptr["sparse_meta"], _stream_handle(stream), ctypes.byref(h), ctypes.byref(info))
    if st:
        _raise(st, info.as_dict())
    return PackedWeight(h, info.as_dict(), dev)


def pack(w: torch.Tensor, bits: torch.Tensor, tile=(128, 128), bit_order: str = "big",
         stream=None) -> PackedWeight:
    """Validate the bit-packed keep mask and compress W (bf16 [n][k] on the GPU)."""
    _check_cuda(w, "w", torch.bfloat16)
    _check_cuda(bits, "bits", torch.uint8)
    n, k = w.shape
    ldw = _row_major_2d(w, "w") if w.numel() else k
    if bits.numel() * 8 < n * k:
        raise ValueError("bits holds fewer than n*k bits")
    if not bits.is_contiguous():
        raise ValueError("bits must be contiguous")
    h = ctypes.c_void_p()
    info = PatchInfo()
    with torch.cuda.device(w.device):
        st = load().patch_pack(ctypes.c_void_p(w.data_ptr()), n, k, ldw, ctypes.c_void_p(bits.data_ptr()),
                               BIT_ORDER[bit_order], int(tile[0]), int(tile[1]), _stream_handle(stream),
                               ctypes.byref(h), ctypes.byref(info))
    if st:
        _raise(st, info.as_dict())
    return PackedWeight(h, info.as_dict(), w.device)


def sample_mask(tile_logits: torch.Tensor, group_logits: torch.Tensor, n: int, k: int, tile=(128, 128),
                kappa: float = 1.0, tile_noise: Optional[torch.Tensor] = None,
                group_noise: Optional[torch.Tensor] = None, bit_order: str = "big",
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Hard sample of a tile configuration as bit-packed mask bits (uint8 [n*k/8] on the GPU).

    tile_logits f32 [tiles][2] (dense, 2:4); group_logits f32 [n][k/4][6]; noise of the same
    shapes or None."""
    tn, tk = int(tile[0]), int(tile[1])
    tiles = (n // tn) * (k // tk) if tn and tk else 0
    shapes = {"tile_logits": (tile_logits, (tiles, 2)), "group_logits": (group_logits, (n, k // 4, 6)),
              "tile_noise": (tile_noise, (tiles, 2)), "group_noise": (group_noise, (n, k // 4, 6))}
    for name, (t, shape) in shapes.items():
        if t is None:
            if name.endswith("logits"):
                raise ValueError(f"{name} is required")
            continue
        _check_cuda(t, name, torch.float32)
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous {shape}, got {tuple(t.shape)}")
    if out is None:
        out = torch.empty(n * k // 8, dtype=torch.uint8, device=tile_logits.device)
    _check_cuda(out, "out", torch.uint8)
    if out.numel() * 8 < n * k:
        raise ValueError("out holds fewer than n*k bits")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    st = load().patch_sample_mask(ptr(tile_logits), ptr(tile_noise), ptr(group_logits), ptr(group_noise), int(n),
                                  int(k), tn, tk, float(kappa), BIT_ORDER[bit_order], ptr(out),
                                  _stream_handle(stream))
    if st:
        _raise(st)
    return out


def mask_unpack(bits: torch.Tensor, count: int, bit_order: str = "big", out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Expand `count` packed mask bits to uint8 0/1 on the GPU."""
    count = int(count)
    if count < 0:
        raise ValueError("count must be >= 0")
    # sizes first: the kernel reads ceil(count/8) bytes of bits and writes count bytes of out
    if bits.numel() * 8 < count or not bits.is_contiguous():
        raise ValueError(f"bits must be contiguous and hold at least {count} bits, got {bits.numel()} bytes")
    if out is not None and (out.numel() < count or not out.is_contiguous()):
        raise ValueError(f"out must be contiguous with at least {count} elements, got {out.numel()}")
    _check_cuda(bits, "bits", torch.uint8)
    if out is None:
        out = torch.empty(count, dtype=torch.uint8, device=bits.device)
    _check_cuda(out, "out", torch.uint8)
    st = load().patch_mask_unpack(ctypes.c_void_p(bits.data_ptr()), int(count), BIT_ORDER[bit_order],
                                  ctypes.c_void_p(out.data_ptr()), _stream_handle(stream))
    if st:
        _raise(st)
    return out
