"""Mask files and packed-weight files.

The method's released artifact is a bit-packed binary keep/prune mask over a
frozen base model, stored as an .npz, and applying it zeroes the pruned weights
("llama_3.2_1b-PATCH-45Sparse" model card, description and "How to use").
This module reads such a file into per-matrix bit arrays, packs the matching
weights with the library (patch_pack), applies the masks (patch_unpack of the
packed weight) and saves / loads packed weights (patch_export / patch_import).

Mask file layout (the card gives no key names or shapes): one array per linear
weight, keyed by the weight's parameter name (a key may also omit the trailing
".weight"); the array holds the mask of the row-major [out][in] weight packed
8 bits to a byte, 1 = keep, either flat (ceil(out*in/8) bytes) or as
[out][in/8].  Bit order MSB first (numpy.packbits' default) unless stated.

Packed-weight file layout (this library's own): an uncompressed .npz with, per
matrix, "<name>::shape" = int64 [n, k, tile_n, tile_k] and "<name>::<array>"
for tile_map, dense_vals, sparse_vals and sparse_meta in the exported format,
plus "__patch_format__" = int64 [1].  Files are read with allow_pickle=False.
"""
from __future__ import annotations

import os
from typing import Dict, Iterable, Optional

import numpy as np
import torch

from . import api

FORMAT_VERSION = 1
SEP = "::"


def read_mask_npz(path: str) -> Dict[str, np.ndarray]:
    """{key: uint8 packed bits (flat)} from a mask .npz; arrays must already be bit-packed uint8."""
    out = {}
    with np.load(path, allow_pickle=False) as z:
        for key in z.files:
            a = z[key]
            if a.dtype != np.uint8:
                raise ValueError(f"mask {key!r}: expected bit-packed uint8, got {a.dtype}")
            out[key] = np.ascontiguousarray(a).reshape(-1)
    return out


def _match(masks: Dict[str, np.ndarray], name: str) -> Optional[str]:
    if name in masks:
        return name
    if name.endswith(".weight") and name[: -len(".weight")] in masks:
        return name[: -len(".weight")]
    return None


def pack_from_masks(weights: Dict[str, torch.Tensor], masks: Dict[str, np.ndarray], tile=(128, 128),
                    bit_order: str = "big", strict: bool = True) -> Dict[str, api.PackedWeight]:
    """Pack every weight (bf16 [out][in] on the GPU) that has a mask; returns {weight name: PackedWeight}.

    strict: a mask that matches no weight, or a bit array too short for its weight, raises."""
    packed, used = {}, set()
    for name, w in weights.items():
        key = _match(masks, name)
        if key is None:
            continue
        bits = masks[key]
        n, k = w.shape
        if bits.size * 8 < n * k:
            raise ValueError(f"mask {key!r} holds {bits.size * 8} bits, weight {name!r} needs {n * k}")
        used.add(key)
        dev_bits = torch.from_numpy(bits).to(w.device)
        packed[name] = api.pack(w, dev_bits, tile=tile, bit_order=bit_order)
    if strict:
        unused = sorted(set(masks) - used)
        if unused:
            raise KeyError(f"masks without a matching weight: {unused[:5]}{' ...' if len(unused) > 5 else ''}")
    return packed


def apply_masks(weights: Dict[str, torch.Tensor], masks: Dict[str, np.ndarray], tile=(128, 128),
                bit_order: str = "big", strict: bool = True) -> Dict[str, torch.Tensor]:
    """The card's "apply the mask": each masked weight with its pruned entries set to +0.0
    (computed on the GPU by packing and unpacking, so every mask must be tile-wise dense / 2:4)."""
    return {name: pw.unpack() for name, pw in pack_from_masks(weights, masks, tile, bit_order, strict).items()}


def save_packed(path: str, packed: Dict[str, api.PackedWeight]) -> None:
    """Write packed weights to an uncompressed .npz (see the module notes for the layout)."""
    arrays = {"__patch_format__": np.array([FORMAT_VERSION], np.int64)}
    for name, pw in packed.items():
        if SEP in name:
            raise ValueError(f"weight name {name!r} contains {SEP!r}")
        ex = pw.export()
        i = pw.info
        arrays[f"{name}{SEP}shape"] = np.array([i["n"], i["k"], i["tile_n"], i["tile_k"]], np.int64)
        for key in api.PACKED_ARRAYS:
            arrays[f"{name}{SEP}{key}"] = ex[key]
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrays)
    os.replace(tmp, path)


def load_packed(path: str, device=None, names: Optional[Iterable[str]] = None) -> Dict[str, api.PackedWeight]:
    """Read packed weights written by save_packed onto `device` (default: the current GPU)."""
    out = {}
    with np.load(path, allow_pickle=False) as z:
        if "__patch_format__" not in z.files or int(z["__patch_format__"][0]) != FORMAT_VERSION:
            raise ValueError(f"{path}: not a packed-weight file of format {FORMAT_VERSION}")
        all_names = sorted({f.split(SEP)[0] for f in z.files if SEP in f})
        for name in (all_names if names is None else names):
            n, k, tn, tk = (int(v) for v in z[f"{name}{SEP}shape"])
            arrays = {key: z[f"{name}{SEP}{key}"] for key in api.PACKED_ARRAYS}
            out[name] = api.import_packed(arrays, n, k, tile=(tn, tk), device=device)
    return out
