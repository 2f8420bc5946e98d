"""Pins for the CPU oracle: hand-worked examples, the pages' printed figures,
library routines, closed forms, invariants and brute force.  No GPU needed."""
import math

import numpy as np
import pytest

import oracle as O
import synthetic as I
from conftest import read_golden

TILES = [(128, 128), (128, 64), (64, 128), (64, 64)]


def _ints_to_bf16(vals):
    """Small integers (|v| <= 256) are exact in bf16: high half of the float32 pattern."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    return (u >> 16).astype(np.uint16)


# ------------------------------------------------------------------ O1 unpack

def test_unpack_hand_byte():
    b = np.array([0b10110000], dtype=np.uint8)
    assert O.unpack_bits(b, 8, "big").tolist() == [1, 0, 1, 1, 0, 0, 0, 0]
    assert O.unpack_bits(b, 8, "little").tolist() == [0, 0, 0, 0, 1, 1, 0, 1]


@pytest.mark.parametrize("order", ["big", "little"])
@pytest.mark.parametrize("count", [1, 7, 8, 13, 64, 1001])
def test_unpack_matches_numpy(order, count):
    rng = np.random.default_rng(count)
    bits = rng.integers(0, 256, size=(count + 7) // 8, dtype=np.uint8)
    ref = np.unpackbits(bits, count=count, bitorder=order)
    assert np.array_equal(O.unpack_bits(bits, count, order), ref)


def test_unpack_ignores_pad_bits():
    a = O.unpack_bits(np.array([0xFF, 0b10000000], dtype=np.uint8), 9, "big")
    b = O.unpack_bits(np.array([0xFF, 0b11111111], dtype=np.uint8), 9, "big")
    assert a.tolist() == b.tolist() == [1] * 9


# ------------------------------------------------------------------ hand-worked golden

def test_hand_example_2x8():
    g = read_golden("hand_tile_2x8.txt")
    n, k, tn, tk = (int(v) for v in g["n k tn tk"])
    w = _ints_to_bf16([[16 * r + c + 1 for c in range(k)] for r in range(n)])
    bits = np.array([int(v, 16) for v in g["bits_msb_first"]], dtype=np.uint8)
    mask = O.unpack_bits(bits, n * k, "big").reshape(n, k)
    p = O.compress(w, mask, tn, tk)
    assert p.tile_map.tolist() == [int(v) for v in g["tile_map"]]
    assert p.tile_slot.tolist() == [int(v) for v in g["tile_slot"]]
    assert np.array_equal(p.dense_vals.reshape(-1), _ints_to_bf16([int(v) for v in g["dense_vals"]]))
    assert np.array_equal(p.sparse_vals.reshape(-1), _ints_to_bf16([int(v) for v in g["sparse_vals"]]))
    assert p.sparse_meta.reshape(-1).tolist() == [int(v, 16) for v in g["sparse_meta"]]
    wm = O.decompress(p, n, k, tn, tk)
    assert np.array_equal(wm, O.masked_weight(w, mask))
    y = O.gemm_ref(_ints_to_bf16(np.ones((1, k))), wm)
    assert y[0].tolist() == [float(v) for v in g["y_ones"]]
    assert O.measured_sparsity(mask) == float(g["sparsity"][0])


def test_hand_2to4_64x64():
    g = read_golden("hand_2to4_64x64.txt")
    n, k, tn, tk = (int(v) for v in g["n k tn tk"])
    pat = np.array([int(v) for v in g["pattern"]], dtype=np.uint8)
    mask = np.tile(pat, (n, k // 4))
    w = I.gen_weight(n, k, I.rng_for(99, 0, I.ROLE_W))
    p = O.compress(w, mask, tn, tk)
    assert p.tile_map.tolist() == [O.SPARSE24]
    meta = p.sparse_meta[0]
    assert meta.shape == (n, int(g["meta_bytes_per_row"][0]))
    assert np.all(meta == int(g["meta_byte"][0], 16))
    vals = p.sparse_vals[0]
    assert vals.shape == (n, int(g["vals_per_row"][0]))
    assert np.array_equal(vals[:, 0::2], w[:, 0::4]) and np.array_equal(vals[:, 1::2], w[:, 1::4])
    assert O.measured_sparsity(mask) == float(g["sparsity"][0])


# ------------------------------------------------------------------ O2 / O3 classify

def test_shape_errors():
    for n, k, tn, tk in [(100, 128, 64, 64), (128, 96, 64, 64), (128, 128, 32, 64), (128, 128, 64, 256)]:
        with pytest.raises(O.ShapeError):
            O.check_shape(n, k, tn, tk)
    O.check_shape(0, 0, 64, 64)
    O.check_shape(13824, 5120, 128, 64)


@pytest.mark.parametrize("tn,tk", TILES)
def test_classify_all_dense_and_all_sparse(tn, tk):
    n, k = 256, 256
    w = I.gen_weight(n, k, I.rng_for(1, 0, I.ROLE_W))
    T = (n // tn) * (k // tk)
    assert O.classify(np.ones((n, k), np.uint8), tn, tk).tolist() == [O.DENSE] * T
    m = I.magnitude_mask(w, np.ones(T, bool), tn, tk)
    assert O.classify(m, tn, tk).tolist() == [O.SPARSE24] * T


@pytest.mark.parametrize("tn,tk", TILES)
def test_classify_single_flip_is_located(tn, tk):
    prob = I.make_problem("flip", 1, 256, 512, tn, tk, frac=0.5, cfg=2)
    rng = np.random.default_rng(7)
    for _ in range(25):
        r, c = int(rng.integers(0, 256)), int(rng.integers(0, 512))
        m = prob.mask.copy()
        m[r, c] ^= 1
        with pytest.raises(O.MaskError) as e:
            O.classify(m, tn, tk)
        tiles_k = 512 // tk
        assert (e.value.tile, e.value.row, e.value.group) == ((r // tn) * tiles_k + c // tk, r % tn, (c % tk) // 4)


def test_classify_mixed_and_degenerate_tiles():
    tn = tk = 64
    m = np.ones((64, 128), np.uint8)
    m[10, 64 + 8:64 + 12] = [1, 0, 1, 0]           # 2:4 group inside a dense tile
    with pytest.raises(O.MaskError) as e:
        O.classify(m, tn, tk)
    assert (e.value.tile, e.value.row, e.value.group) == (1, 10, 2)
    m = np.tile(np.array([0, 1, 1, 0], np.uint8), (64, 32))
    m[5, 0:4] = 1                                  # dense group inside a 2:4 tile
    with pytest.raises(O.MaskError) as e:
        O.classify(m, tn, tk)
    assert (e.value.tile, e.value.row, e.value.group) == (0, 5, 0)
    m = np.tile(np.array([0, 1, 1, 0], np.uint8), (64, 16))
    m[0, 0:4] = 0                                  # all-zero first group: neither type
    with pytest.raises(O.MaskError) as e:
        O.classify(m, tn, tk)
    assert (e.value.tile, e.value.row, e.value.group) == (0, 0, 0)
    m = np.tile(np.array([0, 1, 1, 0], np.uint8), (64, 16))
    m[63, 60:64] = [1, 1, 1, 0]                    # 3 kept in the last group
    with pytest.raises(O.MaskError) as e:
        O.classify(m, tn, tk)
    assert (e.value.tile, e.value.row, e.value.group) == (0, 63, 15)


# ------------------------------------------------------------------ O4-O6 compress / decompress

@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("frac", [0.0, 0.5, 0.9, 1.0])
def test_compress_invariants(tn, tk, frac):
    prob = I.make_problem("inv", 1, 256, 384, tn, tk, frac=frac, cfg=3)
    p = O.compress(prob.w, prob.mask, tn, tk)
    T = (256 // tn) * (384 // tk)
    S = int(p.tile_map.sum())
    D = T - S
    assert S == prob.meta["n_sparse"]
    # pool sizes in closed form
    assert p.dense_vals.nbytes == 2 * D * tn * tk
    assert p.sparse_vals.nbytes == S * tn * tk
    assert p.sparse_meta.nbytes == S * tn * tk // 8
    # slots: a permutation of 0..D-1 / 0..S-1 in row-major order
    assert p.tile_slot[p.tile_map == 0].tolist() == list(range(D))
    assert p.tile_slot[p.tile_map == 1].tolist() == list(range(S))
    # legal 2:4 codes only
    codes = np.concatenate([p.sparse_meta.reshape(-1) & 0xF, p.sparse_meta.reshape(-1) >> 4])
    assert set(codes.tolist()) <= set(O.LEGAL_CODES)
    # round trips, bitwise
    assert np.array_equal(O.decompress(p, 256, 384, tn, tk), O.masked_weight(prob.w, prob.mask))
    assert np.array_equal(O.mask_of(p, 256, 384, tn, tk), prob.mask)
    # sparsity identity: pruned weights = S * tn * tk / 2
    assert int((prob.mask == 0).sum()) == S * tn * tk // 2
    assert O.measured_sparsity(prob.mask) == 0.5 * S / T


def test_pruned_zero_is_positive_zero():
    prob = I.make_problem("z", 1, 128, 128, 64, 64, frac=1.0, cfg=4)
    wm = O.decompress(O.compress(prob.w, prob.mask, 64, 64), 128, 128, 64, 64)
    assert np.all(wm[prob.mask == 0] == 0)        # 0x0000, never 0x8000


def test_tile_size_consistency():
    """A mask learned at 128x128 (card, hyper-parameters) is valid at every hardware tile size."""
    prob = I.make_problem("c", 1, 512, 512, 128, 128, frac=0.5, cfg=5)
    ref_map = O.classify(prob.mask, 128, 128).reshape(4, 4)
    wm_ref = None
    for tn, tk in TILES:
        p = O.compress(prob.w, prob.mask, tn, tk)
        tm = p.tile_map.reshape(512 // tn, 512 // tk)
        assert np.array_equal(tm, np.repeat(np.repeat(ref_map, 128 // tn, 0), 128 // tk, 1))
        wm = O.decompress(p, 512, 512, tn, tk)
        wm_ref = wm if wm_ref is None else wm_ref
        assert np.array_equal(wm, wm_ref)


def test_empty_weight():
    for n, k in [(0, 128), (128, 0), (0, 0)]:
        w = np.zeros((n, k), np.uint16)
        p = O.compress(w, np.ones((n, k), np.uint8), 64, 64)
        assert p.tile_map.size == 0
        assert O.decompress(p, n, k, 64, 64).shape == (n, k)
        y = O.gemm_ref(np.zeros((3, k), np.uint16), w)
        assert y.shape == (3, n) and np.all(y == 0)


# ------------------------------------------------------------------ the pages' figures

def test_pages_sparsity_figures():
    g = read_golden("pages_sparsity.txt")
    # 2:4 everywhere gives exactly 50.00 %
    prob = I.make_problem("all24", 1, 512, 2048, 128, 128, frac=1.0, cfg=6)
    assert round(100 * O.measured_sparsity(prob.mask), 2) == float(g["maskllm_measured_percent"][0])
    # all dense gives 0 % and the tile map is all dense
    prob0 = I.make_problem("dense", 1, 512, 2048, 128, 128, frac=0.0, cfg=6)
    assert 100 * O.measured_sparsity(prob0.mask) == float(g["dense_percent"][0])
    # one LLaMA-3.2-1B layer (128x128 tiles): 3712 tiles.  The measured 44.99 % at a
    # 45 % target is 0.5 * S / T with S = 3340 2:4 tiles; the fraction s = 0.5 f never
    # exceeds the target's 50 % cap and a measured value below the target is reachable.
    T = sum((n // 128) * (k // 128) for n, k in I.LLAMA32_1B.values())
    assert T == 3712
    S = [s for s in range(T + 1) if round(100 * 0.5 * s / T, 2) == float(g["patch_45_measured_percent"][0])]
    assert S == [3340]
    assert abs(100 * 0.5 * S[0] / T - float(g["patch_45_target_percent"][0])) < 0.05


# ------------------------------------------------------------------ O7 GEMM

def test_gemm_matches_brute_force_tiny():
    prob = I.make_problem("tiny", 16, 256, 256, 128, 128, n_sparse=2, cfg=0)
    wm = O.decompress(O.compress(prob.w, prob.mask, 128, 128), 256, 256, 128, 128)
    y = O.gemm_ref(prob.x, wm)
    yb = O.gemm_brute(prob.x, wm)
    assert np.max(np.abs(y - yb) / (1 + np.abs(yb))) < 1e-12


def test_gemm_non_square_orientation():
    prob = I.make_problem("ns", 3, 128, 64, 64, 64, frac=1.0, cfg=7)
    wm = O.masked_weight(prob.w, prob.mask)
    y = O.gemm_ref(prob.x, wm)
    assert y.shape == (3, 128)
    assert np.max(np.abs(y - O.gemm_brute(prob.x, wm))) < 1e-12


def test_gemm_one_hot_rows_exact():
    prob = I.make_problem("oh", 1, 256, 256, 64, 64, frac=0.7, cfg=8)
    wm = O.decompress(O.compress(prob.w, prob.mask, 64, 64), 256, 256, 64, 64)
    ks = np.arange(0, 256, 3)
    x = np.zeros((ks.size, 256), np.uint16)
    x[np.arange(ks.size), ks] = 0x3F80                 # 1.0
    y = O.gemm_ref(x, wm)
    assert np.array_equal(y, O.bf16_to_f64(wm[:, ks]).T)


def test_gemm_ones_counts_kept():
    prob = I.make_problem("ones", 1, 256, 512, 128, 64, frac=0.6, cfg=9)
    ones_w = np.where(prob.mask == 1, np.uint16(0x3F80), np.uint16(0))
    y = O.gemm_ref(np.full((2, 512), 0x3F80, np.uint16), ones_w)
    assert np.array_equal(y[0], prob.mask.sum(axis=1).astype(np.float64))


def test_gemm_all_dense_is_plain_gemm():
    prob = I.make_problem("d", 4, 128, 256, 128, 128, frac=0.0, cfg=10)
    p = O.compress(prob.w, prob.mask, 128, 128)
    wm = O.decompress(p, 128, 256, 128, 128)
    assert np.array_equal(wm, prob.w)
    x64 = I.bf16_bits_to_f32(prob.x).astype(np.float64)
    w64 = I.bf16_bits_to_f32(prob.w).astype(np.float64)
    assert np.array_equal(O.gemm_ref(prob.x, wm), np.matmul(x64, w64.T))


def test_gemm_reference_error_bound():
    """fp64 summation error of the oracle is far inside the 1e-2 tolerance: compare with
    exactly rounded sums (math.fsum) on sampled outputs at K = 13824."""
    rng = np.random.default_rng(11)
    k = 13824
    x = I.gen_x(2, k, rng)
    w = I.gen_weight(3, k, rng)
    y = O.gemm_ref(x, w)
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    for a in range(2):
        for b in range(3):
            prods = xf[a] * wf[b]                       # exact in fp64
            exact = math.fsum(prods.tolist())
            assert abs(y[a, b] - exact) <= k * 2.0 ** -53 * np.abs(prods).sum() + 1e-300


def test_tolerance_function():
    ref = np.array([[0.0, 10.0]])
    assert O.within_tolerance(np.array([[0.009, 10.1]]), ref)
    assert not O.within_tolerance(np.array([[0.02, 10.0]]), ref)
    assert O.rel_error(np.array([[np.nan, 10.0]]), ref) == float("inf")
    assert O.rel_error(np.array([[0.0]]), ref) == float("inf")


# ------------------------------------------------------------------ planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible mistakes in a copy of the oracle's encoding and check that the
    hand-worked fixture rejects each of them."""
    g = read_golden("hand_tile_2x8.txt")
    want_meta = [int(v, 16) for v in g["sparse_meta"]]
    want_vals = [int(v) for v in g["sparse_vals"]]
    n, k, tn, tk = 4, 16, 2, 8
    w = _ints_to_bf16([[16 * r + c + 1 for c in range(k)] for r in range(n)])
    bits = np.array([int(v, 16) for v in g["bits_msb_first"]], dtype=np.uint8)

    def meta_of(order="big", swap_nibbles=False, swap_i=False):
        mask = O.unpack_bits(bits, n * k, order).reshape(n, k)
        try:
            p = O.compress(w, mask, tn, tk)
        except O.MaskError:
            return None, None
        meta = p.sparse_meta.reshape(-1).tolist()
        if swap_nibbles:
            meta = [((b & 0xF) << 4) | (b >> 4) for b in meta]
        if swap_i:
            def sw(c):
                return (c >> 2) | ((c & 3) << 2)
            meta = [sw(b & 0xF) | (sw(b >> 4) << 4) for b in meta]
        vals = [int(v) for v in I.bf16_bits_to_f32(p.sparse_vals.reshape(-1))]
        return meta, vals

    assert meta_of() == (want_meta, want_vals)
    assert meta_of(order="little") != (want_meta, want_vals)      # wrong bit order
    assert meta_of(swap_nibbles=True)[0] != want_meta             # odd group in low nibble
    assert meta_of(swap_i=True)[0] != want_meta                   # i1 | i0 << 2
    # a GEMM that forgets the transpose (square W, so shapes still conform) or drops
    # the mask is caught by the brute-force pin
    prob = I.make_problem("sq", 2, 64, 64, 64, 64, frac=1.0, cfg=12)
    wm = O.masked_weight(prob.w, prob.mask)
    yb = O.gemm_brute(prob.x, wm)
    assert np.max(np.abs(O.gemm_ref(prob.x, wm) - yb)) < 1e-12
    assert np.max(np.abs(O.bf16_to_f64(prob.x) @ O.bf16_to_f64(wm) - yb)) > 1e-3
    assert np.max(np.abs(O.gemm_ref(prob.x, prob.w) - yb)) > 1e-3


# ------------------------------------------------------------------ generators

def test_generators_deterministic_and_valid():
    a = I.make_problem("g", 8, 256, 256, 128, 64, frac=0.5, cfg=13)
    b = I.make_problem("g", 8, 256, 256, 128, 64, frac=0.5, cfg=13)
    assert np.array_equal(a.bits, b.bits) and np.array_equal(a.w, b.w) and np.array_equal(a.x, b.x)
    assert np.array_equal(np.unpackbits(a.bits, count=256 * 256).reshape(256, 256), a.mask)
    # magnitude rule: kept values dominate pruned ones within each group of a 2:4 tile
    mag = np.abs(I.bf16_bits_to_f32(a.w)).reshape(256, 64, 4)
    mk = a.mask.reshape(256, 64, 4)
    sparse_groups = mk.sum(axis=2) == 2
    kept_min = np.where(mk == 1, mag, np.inf).min(axis=2)
    pruned_max = np.where(mk == 0, mag, -np.inf).max(axis=2)
    assert np.all(kept_min[sparse_groups] >= pruned_max[sparse_groups])


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], dtype=np.float32)
    b = I.f32_to_bf16_bits(f)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020]


def test_nonuniform_fractions():
    tiles = [1024] * 4 + [2752] * 3
    f, s = I.nonuniform_fractions(tiles, I.rng_for(4, 0, I.ROLE_FRACTIONS))
    assert sum(s) == round(0.9 * sum(tiles)) == 11117
    assert all(0 <= si <= ti for si, ti in zip(s, tiles))
    assert np.all((f >= 0.3 - 1e-12) & (f <= 1.0 + 1e-12))
