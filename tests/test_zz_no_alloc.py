"""patch_pack_noalloc through the C ABI: the allocation-free variant of patch_pack
(caller-owned pools and handle storage, validation scratch in a per-GPU static
array).  Its packed format must equal patch_pack's and the oracle's bit for bit
and its GEMM must equal patch_pack's bit for bit, on two calls in a row, the
second smaller; an invalid mask is located through the reused scratch, and a
valid call after it packs correctly."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def pack_noalloc(P, prob, bits=None, pools_scale=1.0):
    """Calls patch_pack_noalloc with pools sized for every tile dense / every tile 2:4
    (times pools_scale); returns (status, PackedWeight or None, info)."""
    L = P.load()
    n, k, tn, tk = prob.n, prob.k, prob.tn, prob.tk
    tiles = (n // tn) * (k // tk)
    w = dev_u16(prob.w)
    b = torch.from_numpy(prob.bits if bits is None else bits).cuda()
    keep = {"w": w, "bits": b,
            "tile_map": torch.empty(tiles, dtype=torch.uint8, device="cuda"),
            "tile_desc": torch.empty(tiles, dtype=torch.int32, device="cuda"),
            "dense": torch.empty(int(n * k * pools_scale), dtype=torch.int16, device="cuda"),
            "sparse": torch.empty(int(n * k // 2 * pools_scale), dtype=torch.int16, device="cuda"),
            "meta": torch.empty(int((n * k // 8 + 16) * pools_scale), dtype=torch.uint8, device="cuda"),
            "storage": P.WeightStorage()}
    h = ctypes.c_void_p()
    info = P.PatchInfo()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = L.patch_pack_noalloc(w.data_ptr(), n, k, k, b.data_ptr(), 0, tn, tk, stream,
                              keep["tile_map"].data_ptr(), keep["tile_desc"].data_ptr(),
                              keep["dense"].data_ptr(), keep["dense"].numel() * 2,
                              keep["sparse"].data_ptr(), keep["sparse"].numel() * 2,
                              keep["meta"].data_ptr(), keep["meta"].numel(),
                              ctypes.byref(keep["storage"]), ctypes.byref(h), ctypes.byref(info))
    if st:
        return st, None, info
    pw = P.PackedWeight(h, info.as_dict(), w.device)
    pw._keep = keep  # the caller owns the pools and the handle storage
    return st, pw, info


def check_same_as_pack(P, prob):
    st, pw, info = pack_noalloc(P, prob)
    assert st == 0, P.load().patch_last_error()
    ref = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(prob.tn, prob.tk))
    assert pw.info == ref.info
    got, want = pw.export(), ref.export()
    oracle = O.compress(prob.w, prob.mask, prob.tn, prob.tk)
    for key in ("tile_map", "tile_slot", "dense_vals", "sparse_vals", "sparse_meta"):
        assert np.array_equal(got[key], want[key]), key
        assert np.array_equal(got[key], getattr(oracle, key)), key
    x = dev_u16(prob.x)
    for kern in ("auto", "stream") if prob.m <= 16 else ("auto", "tiled"):
        assert torch.equal(pw.gemm(x, kernel=kern), ref.gemm(x, kernel=kern)), kern
    assert torch.equal(pw.unpack(), ref.unpack())
    torch.cuda.synchronize()


def test_two_calls_in_a_row_second_smaller(P):
    big = I.make_problem("na1", 300, 1024, 768, 128, 64, frac=0.7, cfg=90)
    small = I.make_problem("na2", 16, 256, 256, 64, 64, frac=0.5, cfg=91)
    check_same_as_pack(P, big)
    check_same_as_pack(P, small)


def test_invalid_mask_then_valid_call(P):
    prob = I.make_problem("na3", 64, 512, 512, 64, 128, frac=0.8, cfg=92)
    mask = prob.mask.copy()
    sp = np.flatnonzero(prob.tile_sparse)
    t = int(sp[len(sp) // 2])
    ti, tj = divmod(t, 512 // 128)
    r, c = ti * 64 + 9, tj * 128 + 4 * 7 + 1
    mask[r, c] ^= 1
    st, pw, info = pack_noalloc(P, prob, bits=I.pack_mask_bits(mask))
    assert st == 3 and pw is None
    with pytest.raises(O.MaskError) as e:
        O.classify(mask, 64, 128)
    assert (info.bad_tile, info.bad_row, info.bad_group) == (e.value.tile, e.value.row, e.value.group)
    check_same_as_pack(P, prob)  # the scratch's error word was reset


def test_pools_too_small(P):
    prob = I.make_problem("na4", 16, 256, 512, 64, 64, frac=0.25, cfg=93)
    st, pw, _ = pack_noalloc(P, prob, pools_scale=0.25)
    assert st == 1 and pw is None
    assert b"pools too small" in P.load().patch_last_error()
