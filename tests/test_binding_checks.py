"""CPU tests of the binding's buffer checks: undersized or mis-shaped buffers are
refused with ValueError before anything reaches the library (no GPU needed,
no kernel is launched)."""
import numpy as np
import pytest
import torch

from sparse_gemm_patch_amd import api


def _fake_weight(n, k):
    info = {"n": n, "k": k, "tile_n": 128, "tile_k": 128}
    return api.PackedWeight(None, info, torch.device("cpu"))


@pytest.mark.parametrize("shape", [(255, 256), (256, 128), (128, 256), (256 * 256,)])
def test_unpack_out_shape(shape):
    pw = _fake_weight(256, 256)
    with pytest.raises(ValueError, match="out must be"):
        pw.unpack(out=torch.empty(shape, dtype=torch.bfloat16))


@pytest.mark.parametrize("nbytes,count", [(1, 9), (0, 1), (2, 17)])
def test_mask_unpack_short_bits(nbytes, count):
    with pytest.raises(ValueError, match="bits"):
        api.mask_unpack(torch.zeros(nbytes, dtype=torch.uint8), count)


def test_mask_unpack_short_out():
    with pytest.raises(ValueError, match="out"):
        api.mask_unpack(torch.zeros(4, dtype=torch.uint8), 32, out=torch.empty(31, dtype=torch.uint8))


def test_mask_unpack_negative_count():
    with pytest.raises(ValueError, match="count"):
        api.mask_unpack(torch.zeros(4, dtype=torch.uint8), -1)


def _arrays(tiles, nd, ns, tn=128, tk=128):
    tm = np.array([0] * nd + [1] * ns, np.uint8)
    assert tm.size == tiles
    return {"tile_map": tm, "dense_vals": np.zeros(nd * tn * tk, np.uint16),
            "sparse_vals": np.zeros(ns * tn * tk // 2, np.uint16),
            "sparse_meta": np.full(ns * tn * tk // 8, 0x44, np.uint8)}


def test_import_tile_map_disagrees_with_shape():
    """A file whose shape entry says 256x256 (4 tiles) but whose tile map holds 2."""
    arrs = _arrays(2, 1, 1)
    with pytest.raises(ValueError, match="tile_map has 2 entries"):
        api.import_packed(arrs, 256, 256, tile=(128, 128))
    arrs = _arrays(8, 4, 4)
    with pytest.raises(ValueError, match="tile_map has 8 entries"):
        api.import_packed(arrs, 256, 256, tile=(128, 128))


@pytest.mark.parametrize("n,k,tile", [(200, 256, (128, 128)), (256, 256, (96, 128)), (256, 192, (128, 128))])
def test_import_shape_not_whole_tiles(n, k, tile):
    with pytest.raises(ValueError, match="whole number"):
        api.import_packed(_arrays(4, 4, 0), n, k, tile=tile)


def test_import_pool_size_mismatch():
    arrs = _arrays(4, 2, 2)
    arrs["sparse_vals"] = arrs["sparse_vals"][:-1]
    with pytest.raises(ValueError, match="sparse_vals"):
        api.import_packed(arrs, 256, 256, tile=(128, 128))
