"""GPU tests of mask-file ingestion and packed-weight files (patch_import).

* patch_import of the oracle's compressed arrays builds a weight whose export
  is those arrays bit for bit, and whose GEMM matches the oracle and, bit for
  bit, the GEMM of the same weight packed from W and the mask;
* save_packed / load_packed round-trips several matrices of every tile shape;
* pack_from_masks / apply_masks over a small synthetic model's mask .npz give
  what per-matrix packing and the oracle's masked weight give.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu

TILES = [(128, 128), (128, 64), (64, 128), (64, 64)]


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_arrays(prob):
    ref = O.compress(prob.w, prob.mask, prob.tn, prob.tk)
    return {"tile_map": ref.tile_map, "tile_slot": ref.tile_slot, "dense_vals": ref.dense_vals,
            "sparse_vals": ref.sparse_vals, "sparse_meta": ref.sparse_meta}


@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("frac", [0.0, 0.6, 1.0])
def test_import_of_oracle_arrays(P, tn, tk, frac):
    prob = I.make_problem("imp", 150, 384, 512, tn, tk, frac=frac, cfg=71)
    arrs = oracle_arrays(prob)
    pw = P.import_packed(arrs, prob.n, prob.k, tile=(tn, tk))
    got = pw.export()
    for key in ("tile_map", "tile_slot", "dense_vals", "sparse_vals", "sparse_meta"):
        assert np.array_equal(got[key], arrs[key]), key
    x = dev_u16(prob.x)
    pw2 = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(tn, tk))
    for kernel in ("auto", "stream" if prob.m <= 16 else "tiled"):
        y = pw.gemm(x, out_dtype=torch.float32, kernel=kernel)
        y2 = pw2.gemm(x, out_dtype=torch.float32, kernel=kernel)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y.cpu().numpy().astype(np.float64), ref) <= 1e-4
    assert np.array_equal(host_u16(pw.unpack()), O.masked_weight(prob.w, prob.mask))


def test_import_decode_kernel(P):
    prob = I.make_problem("impd", 7, 512, 1024, 128, 128, frac=0.9, cfg=72)
    pw = P.import_packed(oracle_arrays(prob), prob.n, prob.k, tile=(128, 128))
    y = pw.gemm(dev_u16(prob.x), out_dtype=torch.float32, kernel="stream")
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y.cpu().numpy().astype(np.float64), ref) <= 1e-4


def test_import_rejects_bad_code_like_the_header_says(P):
    prob = I.make_problem("impbad", 1, 256, 256, 64, 64, frac=1.0, cfg=73)
    arrs = oracle_arrays(prob)
    arrs["sparse_meta"] = arrs["sparse_meta"].copy()
    arrs["sparse_meta"][5, 3, 2] = (arrs["sparse_meta"][5, 3, 2] & 0xF0) | 0x3  # group 4: i0 = 3, i1 = 0
    with pytest.raises(P.PatchError) as e:
        P.import_packed(arrs, prob.n, prob.k, tile=(64, 64))
    assert e.value.status_name == "PATCH_E_MASK"
    assert (e.value.info["bad_tile"], e.value.info["bad_row"], e.value.info["bad_group"]) == (5, 3, 4)


def test_save_and_load_packed(P, tmp_path):
    from sparse_gemm_patch_amd import checkpoint as C
    probs = {f"layer.{i}.proj.weight": I.make_problem("ck", 64, 256 + 128 * (i % 2), 384, tn, tk,
                                                       frac=0.25 * i, cfg=74, matrix=i)
             for i, (tn, tk) in enumerate(TILES)}
    packed = {name: P.pack(dev_u16(p.w), torch.from_numpy(p.bits).cuda(), tile=(p.tn, p.tk))
              for name, p in probs.items()}
    path = str(tmp_path / "packed.npz")
    C.save_packed(path, packed)
    loaded = C.load_packed(path)
    assert set(loaded) == set(packed)
    for name, p in probs.items():
        a, b = packed[name].export(), loaded[name].export()
        for key in a:
            assert np.array_equal(a[key], b[key]), (name, key)
        assert loaded[name].info == packed[name].info
        x = dev_u16(p.x)
        assert torch.equal(packed[name].gemm(x), loaded[name].gemm(x))
    sub = C.load_packed(path, names=["layer.2.proj.weight"])
    assert list(sub) == ["layer.2.proj.weight"]


def test_mask_npz_ingestion(P, tmp_path):
    """A synthetic model's masks in one .npz: pack and apply, per matrix."""
    from sparse_gemm_patch_amd import checkpoint as C
    shapes = {"q_proj": (256, 256), "k_proj": (128, 256), "gate_proj": (512, 256), "down_proj": (256, 512)}
    probs, weights, npz = {}, {}, {}
    for i, (mod, (n, k)) in enumerate(shapes.items()):
        name = f"model.layers.0.{mod}.weight"
        p = I.make_problem(mod, 1, n, k, 128, 128, frac=0.9, cfg=75, matrix=i)
        probs[name] = p
        weights[name] = dev_u16(p.w)
        # the row-packed form for one of them, the flat form for the rest; one key without ".weight"
        key = name if i % 2 == 0 else name[: -len(".weight")]
        npz[key] = np.packbits(p.mask.astype(np.uint8), axis=1) if i == 1 else p.bits
    weights["model.layers.0.o_proj.weight"] = dev_u16(np.zeros((256, 256), np.uint16))  # no mask: stays dense
    path = str(tmp_path / "mask.npz")
    np.savez(path, **npz)
    masks = C.read_mask_npz(path)
    packed = C.pack_from_masks(weights, masks)
    assert set(packed) == set(probs)
    applied = C.apply_masks(weights, masks)
    for name, p in probs.items():
        ref = O.compress(p.w, p.mask, 128, 128)
        assert np.array_equal(packed[name].export()["sparse_meta"], ref.sparse_meta)
        assert np.array_equal(host_u16(applied[name]), O.masked_weight(p.w, p.mask))
    with pytest.raises(KeyError):
        C.pack_from_masks({k: v for k, v in weights.items() if "q_proj" not in k}, masks)
    short = dict(masks)
    key = next(k for k in short if "gate_proj" in k)
    short[key] = short[key][:10]
    with pytest.raises(ValueError):
        C.pack_from_masks(weights, short)
