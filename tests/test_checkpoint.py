"""Mask-file reading (no GPU): the .npz forms the loader accepts and rejects."""
import numpy as np
import pytest

from sparse_gemm_patch_amd import checkpoint as C
import synthetic as I


def test_flat_and_row_packed_masks_read_the_same(tmp_path):
    prob = I.make_problem("npz", 1, 128, 256, 64, 64, frac=0.5, cfg=70)
    flat = prob.bits
    rows = np.packbits(prob.mask.astype(np.uint8), axis=1)  # [out][in/8]
    path = tmp_path / "mask.npz"
    np.savez(path, **{"model.layers.0.mlp.up_proj.weight": flat, "model.layers.0.mlp.down_proj": rows})
    m = C.read_mask_npz(str(path))
    assert set(m) == {"model.layers.0.mlp.up_proj.weight", "model.layers.0.mlp.down_proj"}
    assert np.array_equal(m["model.layers.0.mlp.up_proj.weight"], flat)
    assert np.array_equal(m["model.layers.0.mlp.down_proj"], flat)  # same bytes when in % 8 == 0


def test_unpacked_masks_are_rejected(tmp_path):
    path = tmp_path / "mask.npz"
    np.savez(path, a=np.ones((4, 8), bool))
    with pytest.raises(ValueError):
        C.read_mask_npz(str(path))


def test_name_matching():
    masks = {"a.weight": np.zeros(1, np.uint8), "b": np.zeros(1, np.uint8)}
    assert C._match(masks, "a.weight") == "a.weight"
    assert C._match(masks, "b.weight") == "b"
    assert C._match(masks, "c.weight") is None


def test_packed_file_needs_the_format_marker(tmp_path):
    path = tmp_path / "x.npz"
    np.savez(path, **{"q::shape": np.array([64, 64, 64, 64], np.int64)})
    with pytest.raises(ValueError):
        C.load_packed(str(path))


def test_packed_file_shape_disagrees_with_tile_map(tmp_path):
    """A packed file whose shape entry (256x256: 4 tiles of 128x128) disagrees with its
    tile map (2 entries) is refused on the host before the library reads anything."""
    path = tmp_path / "bad.npz"
    arrays = {"__patch_format__": np.array([C.FORMAT_VERSION], np.int64),
              "q::shape": np.array([256, 256, 128, 128], np.int64),
              "q::tile_map": np.array([0, 1], np.uint8),
              "q::dense_vals": np.zeros(128 * 128, np.uint16),
              "q::sparse_vals": np.zeros(128 * 64, np.uint16),
              "q::sparse_meta": np.full(128 * 16, 0x44, np.uint8)}
    np.savez(path, **arrays)
    with pytest.raises(ValueError, match="tile_map has 2 entries"):
        C.load_packed(str(path))
