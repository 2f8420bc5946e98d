"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Packing, unpacking and mask expansion must be bit-exact; Y must satisfy
|Y - Y_ref| <= 1e-2 (1 + |Y_ref|) elementwise with no NaN/Inf, Y_ref the fp64
oracle.  Exact closed forms (one-hot rows, all-ones) must match with zero
tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu

TILES = [(128, 128), (128, 64), (64, 128), (64, 64)]
TOL = 1e-2


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    """numpy uint16 bf16 bits -> torch bf16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def y_host(y):
    return y.float().cpu().numpy().astype(np.float64)


def pack_problem(P, prob, order="big"):
    bits = prob.bits if order == "big" else I.pack_mask_bits(prob.mask, "little")
    return P.pack(dev_u16(prob.w), dev_u8(bits), tile=(prob.tn, prob.tk), bit_order=order)


def check_packed(pw, prob):
    ref = O.compress(prob.w, prob.mask, prob.tn, prob.tk)
    got = pw.export()
    assert np.array_equal(got["tile_map"], ref.tile_map)
    assert np.array_equal(got["tile_slot"], ref.tile_slot)
    assert np.array_equal(got["dense_vals"], ref.dense_vals)
    assert np.array_equal(got["sparse_vals"], ref.sparse_vals)
    assert np.array_equal(got["sparse_meta"], ref.sparse_meta)
    return ref


# ------------------------------------------------------------------ mask unpack

@pytest.mark.parametrize("order", ["big", "little"])
@pytest.mark.parametrize("count", [1, 7, 8, 9, 1000, 65536 + 3])
def test_mask_unpack_bit_exact(P, order, count):
    rng = np.random.default_rng(count)
    bits = rng.integers(0, 256, size=(count + 7) // 8, dtype=np.uint8)
    out = P.mask_unpack(dev_u8(bits), count, order).cpu().numpy()
    assert np.array_equal(out, O.unpack_bits(bits, count, order))


# ------------------------------------------------------------------ pack / unpack

@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("frac", [0.0, 0.3, 0.9, 1.0])
def test_pack_bit_exact(P, tn, tk, frac):
    prob = I.make_problem("pack", 1, 512, 768, tn, tk, frac=frac, cfg=20)
    pw = pack_problem(P, prob)
    ref = check_packed(pw, prob)
    S = int(ref.tile_map.sum())
    T = ref.tile_map.size
    assert pw.info["n_sparse"] == S and pw.info["n_dense"] == T - S
    assert pw.info["sparsity"] == 0.5 * S / T == O.measured_sparsity(prob.mask)
    wm = host_u16(pw.unpack())
    assert np.array_equal(wm, O.decompress(ref, 512, 768, tn, tk))
    assert np.array_equal(wm, O.masked_weight(prob.w, prob.mask))


def test_pack_lsb_first_and_strided_w(P):
    prob = I.make_problem("lsb", 1, 256, 512, 64, 128, frac=0.5, cfg=21)
    wide = np.zeros((256, 512 + 64), np.uint16)
    wide[:, :512] = prob.w
    w_dev = dev_u16(wide)[:, :512]
    bits = I.pack_mask_bits(prob.mask, "little")
    pw = P.pack(w_dev, dev_u8(bits), tile=(64, 128), bit_order="little")
    check_packed(pw, prob)
    out = torch.zeros((256, 512 + 128), dtype=torch.bfloat16, device="cuda")
    pw.unpack(out=out[:, :512])
    got = host_u16(out)
    assert np.array_equal(got[:, :512], O.masked_weight(prob.w, prob.mask))
    assert np.all(got[:, 512:] == 0)  # columns past K untouched


@pytest.mark.parametrize("tn,tk", TILES)
def test_invalid_mask_located_like_the_oracle(P, tn, tk):
    prob = I.make_problem("bad", 1, 256, 512, tn, tk, frac=0.6, cfg=22)
    rng = np.random.default_rng(5)
    cases = [(int(rng.integers(0, 256)), int(rng.integers(0, 512))) for _ in range(6)] + [(255, 511), (0, 0)]
    for r, c in cases:
        m = prob.mask.copy()
        m[r, c] ^= 1
        with pytest.raises(O.MaskError) as want:
            O.classify(m, tn, tk)
        with pytest.raises(P.PatchError) as got:
            P.pack(dev_u16(prob.w), dev_u8(I.pack_mask_bits(m)), tile=(tn, tk))
        assert got.value.status_name == "PATCH_E_MASK"
        gi = got.value.info
        assert (gi["bad_tile"], gi["bad_row"], gi["bad_group"]) == (want.value.tile, want.value.row, want.value.group)


def test_two_errors_report_the_first(P):
    prob = I.make_problem("bad2", 1, 256, 256, 64, 64, frac=0.5, cfg=23)
    m = prob.mask.copy()
    m[200, 250] ^= 1
    m[70, 3] ^= 1
    with pytest.raises(O.MaskError) as want:
        O.classify(m, 64, 64)
    with pytest.raises(P.PatchError) as got:
        P.pack(dev_u16(prob.w), dev_u8(I.pack_mask_bits(m)), tile=(64, 64))
    gi = got.value.info
    assert (gi["bad_tile"], gi["bad_row"], gi["bad_group"]) == (want.value.tile, want.value.row, want.value.group)


def test_shape_and_argument_errors(P):
    w = torch.zeros((192, 128), dtype=torch.bfloat16, device="cuda")
    bits = torch.zeros(192 * 128 // 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PatchError) as e:
        P.pack(w, bits, tile=(128, 128))
    assert e.value.status_name == "PATCH_E_SHAPE"
    with pytest.raises(P.PatchError) as e:
        P.pack(w, bits, tile=(64, 32))
    assert e.value.status_name == "PATCH_E_SHAPE"


def test_allocation_failure_is_clean(P, monkeypatch):
    prob = I.make_problem("nomem", 1, 256, 256, 64, 64, frac=0.5, cfg=24)
    w, bits = dev_u16(prob.w), dev_u8(prob.bits)
    for nth in (1, 2, 3, 4, 5, 6):  # scratch, tile map, descriptors, dense, 2:4 values, codes
        monkeypatch.setenv("PATCH_TEST_FAIL_ALLOC", str(nth))
        with pytest.raises(P.PatchError) as e:
            P.pack(w, bits, tile=(64, 64))
        assert e.value.status_name == "PATCH_E_NOMEM"
    monkeypatch.delenv("PATCH_TEST_FAIL_ALLOC")
    check_packed(P.pack(w, bits, tile=(64, 64)), prob)


def test_empty_weights(P):
    for n, k in [(0, 128), (128, 0)]:
        w = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
        bits = torch.zeros(max(1, n * k // 8), dtype=torch.uint8, device="cuda")
        pw = P.pack(w, bits, tile=(64, 64))
        assert pw.info["n_dense"] == pw.info["n_sparse"] == 0
        x = torch.randn((5, k), device="cuda").to(torch.bfloat16)
        y = pw.gemm(x, out_dtype=torch.float32)
        assert tuple(y.shape) == (5, n) and (n == 0 or bool(torch.all(y == 0)))


# ------------------------------------------------------------------ GEMM parity

def gemm_case(P, prob, kernel="auto", out_dtype=torch.bfloat16):
    pw = pack_problem(P, prob)
    y = pw.gemm(dev_u16(prob.x), out_dtype=out_dtype, kernel=kernel)
    torch.cuda.synchronize()
    wm = O.masked_weight(prob.w, prob.mask)
    ref = O.gemm_ref(prob.x, wm)
    return y_host(y), ref


def test_tiny_config(P):
    """W 256x256, 128x128 tiles, 2 dense + 2 2:4 tiles chosen by seed, X 16x256."""
    prob = I.make_problem("tiny", 16, 256, 256, 128, 128, n_sparse=2, cfg=0)
    for kernel in ("auto", "stream", "tiled"):
        for dt in (torch.bfloat16, torch.float32):
            y, ref = gemm_case(P, prob, kernel, dt)
            assert O.rel_error(y, ref) <= TOL, (kernel, dt)


@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("m", [1, 8, 16, 17, 130, 300])
@pytest.mark.parametrize("frac", [0.0, 0.5, 1.0])
def test_gemm_matches_oracle(P, tn, tk, m, frac):
    prob = I.make_problem("g", m, 384, 640, tn, tk, frac=frac, cfg=30 + m)
    for dt in (torch.bfloat16, torch.float32):
        y, ref = gemm_case(P, prob, "auto", dt)
        err = O.rel_error(y, ref)
        assert err <= TOL, (dt, err)
        if dt == torch.float32:
            assert err <= 1e-4, err  # fp32 output: only accumulation-order error


@pytest.mark.parametrize("kernel", ["stream", "tiled"])
def test_one_hot_rows_exact(P, kernel):
    prob = I.make_problem("oh", 16, 256, 512, 64, 128, frac=0.7, cfg=40)
    ks = (np.arange(16) * 31 + 5) % 512
    x = np.zeros((16, 512), np.uint16)
    x[np.arange(16), ks] = 0x3F80
    pw = pack_problem(P, prob)
    y = pw.gemm(dev_u16(x), kernel=kernel)
    wm = O.masked_weight(prob.w, prob.mask)
    assert np.array_equal(host_u16(y), wm[:, ks].T)  # bf16 bits, zero tolerance


@pytest.mark.parametrize("kernel,m", [("stream", 16), ("tiled", 200)])
def test_ones_count_kept_exactly(P, kernel, m):
    prob = I.make_problem("ones", m, 256, 1024, 128, 64, frac=0.6, cfg=41)
    w1 = np.full_like(prob.w, 0x3F80)
    pw = P.pack(dev_u16(w1), dev_u8(prob.bits), tile=(128, 64))
    y = pw.gemm(dev_u16(np.full((m, 1024), 0x3F80, np.uint16)), out_dtype=torch.float32, kernel=kernel)
    want = prob.mask.sum(axis=1).astype(np.float64)
    assert np.array_equal(y_host(y), np.broadcast_to(want, (m, 256)))


@pytest.mark.parametrize("k", [64, 192, 1088, 2048, 4160])
@pytest.mark.parametrize("m", [1, 5, 16, 40, 100])
def test_stream_k_ranges_and_determinism(P, k, m):
    """16 waves (8 with more than 32 rows) share the K chunks of a block: fewer chunks than waves,
    a ragged last round, many rounds."""
    prob = I.make_problem("sk", m, 512, k, 128, 64, frac=0.5, cfg=42)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    y1 = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
    y2 = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)  # bitwise run-to-run
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(y1), ref) <= 1e-4


@pytest.mark.parametrize("block_m", [256, 192, 128, 64])
@pytest.mark.parametrize("tn,tk,frac", [(128, 128, 0.5), (64, 64, 0.9), (128, 64, 0.0), (64, 128, 1.0)])
def test_tiled_block_rows(P, block_m, tn, tk, frac):
    """Every block height of the tiled kernel: ragged M (300 rows) and N (640 = 2.5 blocks of 256)."""
    prob = I.make_problem("bm", 300, 640, 1024, tn, tk, frac=frac, cfg=48)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    y32 = pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=block_m)
    y16 = pw.gemm(x, out_dtype=torch.bfloat16, kernel="tiled", block_m=block_m)
    assert O.rel_error(y_host(y32), ref) <= 1e-4
    assert O.rel_error(y_host(y16), ref) <= TOL
    # bf16 Y leaves through an LDS staging buffer, fp32 Y straight from the
    # accumulators: the two must agree to the last bit after rounding
    assert torch.equal(y16, y32.to(torch.bfloat16))


@pytest.mark.parametrize("tn,tk,k", [(64, 64, 4224), (128, 128, 8448)])
def test_tiled_more_than_64_tile_columns(P, tn, tk, k):
    """66 tile columns: the tiled kernel holds descriptors 64 columns at a time and must move
    to the next window in the middle of a block."""
    prob = I.make_problem("win", 300, 256, k, tn, tk, frac=0.5, cfg=52)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    ys = [pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=b) for b in (256, 192, 128, 64)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(ys[0]), ref) <= 1e-4


@pytest.mark.parametrize("m,n", [(5500, 640), (4096, 1024), (4096, 512)])
def test_tiled_64_rows_every_kernel(P, m, n):
    """64-row blocks run on two-per-CU k_gemm_tiled workgroups when 256-row-wide blocks give more
    than 256 workgroups (5500 x 640: 3 x 86), on the warp-specialised kernel when they give at most
    256 (4096 x 1024: 4 x 64), and on its 128-row-wide form when they give at most 128
    (4096 x 512: 2 x 64)."""
    prob = I.make_problem("bm64", m, n, 512, 128, 64, frac=0.6, cfg=51)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    y32 = pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=64)
    y16 = pw.gemm(x, out_dtype=torch.bfloat16, kernel="tiled", block_m=64)
    y256 = pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=256)
    torch.cuda.synchronize()
    assert torch.equal(y32, y256)  # same K order in every block height
    assert torch.equal(y16, y32.to(torch.bfloat16))
    rows = np.r_[0:70, m - 70:m]
    ref = O.gemm_ref(prob.x[rows], O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(y32)[rows], ref) <= 1e-4


@pytest.mark.parametrize("block_m", [256, 192, 128, 64])
def test_tiled_block_rows_one_hot_exact(P, block_m):
    prob = I.make_problem("bmoh", 200, 256, 512, 64, 128, frac=0.7, cfg=49)
    ks = (np.arange(200) * 37 + 11) % 512
    x = np.zeros((200, 512), np.uint16)
    x[np.arange(200), ks] = 0x3F80
    pw = pack_problem(P, prob)
    y = pw.gemm(dev_u16(x), kernel="tiled", block_m=block_m)
    assert np.array_equal(host_u16(y), O.masked_weight(prob.w, prob.mask)[:, ks].T)


def test_tiled_block_rows_rejects_other_values(P):
    prob = I.make_problem("bmbad", 32, 128, 128, 64, 64, frac=0.5, cfg=50)
    pw = pack_problem(P, prob)
    with pytest.raises(P.PatchError) as e:
        pw.gemm(dev_u16(prob.x), kernel="tiled", block_m=96)
    assert e.value.status_name == "PATCH_E_INVALID_ARG"


def test_strided_x_and_y(P):
    prob = I.make_problem("ld", 40, 256, 512, 64, 64, frac=0.5, cfg=43)
    pw = pack_problem(P, prob)
    xw = torch.zeros((40, 512 + 64), dtype=torch.bfloat16, device="cuda")
    xw[:, :512] = dev_u16(prob.x)
    yw = torch.full((40, 256 + 8), 7.0, dtype=torch.float32, device="cuda")
    pw.gemm(xw[:, :512], out=yw[:, :256], out_dtype=torch.float32)
    got = y_host(yw)
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(got[:, :256], ref) <= TOL
    assert np.all(got[:, 256:] == 7.0)  # padding columns untouched


def test_gemm_m_zero_is_noop(P):
    prob = I.make_problem("m0", 1, 128, 128, 64, 64, frac=0.5, cfg=44)
    pw = pack_problem(P, prob)
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    assert tuple(pw.gemm(x).shape) == (0, 128)


def test_ldx_limit(P):
    """X rows farther apart than PATCH_MAX_LDX elements are refused, not mis-addressed."""
    prob = I.make_problem("ldxmax", 2, 128, 128, 64, 64, frac=0.5, cfg=45)
    pw = pack_problem(P, prob)
    lib = P.load()
    y = torch.empty((2, 128), dtype=torch.bfloat16, device="cuda")
    x = dev_u16(prob.x)
    st = lib.patch_gemm(pw._h, x.data_ptr(), 1, (1 << 22) + 8, y.data_ptr(), 128, 0, None)
    assert P.STATUS[st] == "PATCH_E_INVALID_ARG"
    assert b"exceeds" in lib.patch_last_error()


@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("m", [17, 32, 33, 64, 65, 100, 128])
def test_stream_batched_matches_oracle(P, tn, tk, m):
    """The streaming kernel with 2, 4 or 8 blocks of 16 X rows per wave: every tile size, ragged m,
    all-dense, mixed and all-2:4 weights; bf16 Y is the fp32 Y rounded to nearest even; run to run
    bitwise."""
    for frac in (0.0, 0.5, 1.0):
        prob = I.make_problem("sb", m, 384, 640, tn, tk, frac=frac, cfg=90 + m)
        pw = pack_problem(P, prob)
        x = dev_u16(prob.x)
        y32 = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
        y32b = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
        y16 = pw.gemm(x, out_dtype=torch.bfloat16, kernel="stream")
        torch.cuda.synchronize()
        ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
        assert O.rel_error(y_host(y32), ref) <= 1e-4, frac
        assert O.rel_error(y_host(y16), ref) <= TOL, frac
        assert torch.equal(y32, y32b), frac
        assert torch.equal(y16, y32.to(torch.bfloat16)), frac


@pytest.mark.parametrize("n,m,rows", [(256, 32, 16), (256, 128, 64), (5120, 128, 16), (10240, 100, 16)])
def test_stream_rows_independent_of_batch(P, n, m, rows):
    """A product's Y depends on how many waves split K, not on how many X blocks a wave carries:
    16 waves for one W block and up to 32 rows, 8 otherwise.  So a slice of a batched product run
    alone, with the same wave count, equals that slice of the batch bit for bit (256 rows of W: one
    W block, 16-row slices of 32 rows and 64-row slices of 128; 5120 and 10240 rows: 2 and 4 W
    blocks, 8 waves for every m)."""
    prob = I.make_problem("sr", m, n, 1088, 128, 64, frac=0.6, cfg=95)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    y = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
    for r0 in range(0, m, rows):
        ys = pw.gemm(x[r0:r0 + rows].contiguous(), out_dtype=torch.float32, kernel="stream")
        torch.cuda.synchronize()
        assert torch.equal(y[r0:r0 + rows], ys), r0


@pytest.mark.parametrize("n", [5120, 10240])
@pytest.mark.parametrize("tn,tk", TILES)
@pytest.mark.parametrize("m", [1, 16, 24, 64, 128])
def test_stream_w_blocks_match_oracle(P, n, tn, tk, m):
    """Wide weights stream 2 (5120 rows) or 4 (10240 rows) 16-row W blocks per workgroup, every
    block meeting each X copy: every tile size (a 4-block group fills a 64-row tile), decode and
    batched m, all-dense, mixed and all-2:4 weights, K of 6 chunks (fewer than the waves)."""
    for frac in (0.0, 0.5, 1.0):
        prob = I.make_problem("sw", m, n, 384, tn, tk, frac=frac, cfg=98 + m)
        pw = pack_problem(P, prob)
        x = dev_u16(prob.x)
        y32 = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
        y16 = pw.gemm(x, out_dtype=torch.bfloat16, kernel="stream")
        torch.cuda.synchronize()
        ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
        assert O.rel_error(y_host(y32), ref) <= 1e-4, frac
        assert torch.equal(y16, y32.to(torch.bfloat16)), frac
        if m <= 16:
            ya = pw.gemm(x, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(ya, y32), frac


def test_stream_rejects_more_than_128_rows(P):
    prob = I.make_problem("s129", 129, 128, 128, 64, 64, frac=0.5, cfg=96)
    pw = pack_problem(P, prob)
    with pytest.raises(P.PatchError) as e:
        pw.gemm(dev_u16(prob.x), kernel="stream")
    assert e.value.status_name == "PATCH_E_INVALID_ARG"


@pytest.mark.parametrize("n,k,m,want", [(1024, 8192, 64, "stream"), (16384, 1024, 128, "tiled"),
                                        (10240, 2048, 32, "stream")])
def test_auto_kernel_for_small_batches(P, n, k, m, want):
    """Between 17 and 128 rows AUTO estimates both kernels: a narrow weight with a long K streams
    (the tiled kernel would give it 8 workgroups of 128 K steps), a wide one with a short K stays
    tiled at 128 rows (streaming would copy all 128 rows of X for each of its 256 workgroups), and
    streams at 32 rows with 4 W blocks per workgroup."""
    prob = I.make_problem("am", m, n, k, 128, 128, frac=0.9, cfg=97)
    pw = pack_problem(P, prob)
    x = dev_u16(prob.x)
    ya = pw.gemm(x, out_dtype=torch.float32)
    ys = pw.gemm(x, out_dtype=torch.float32, kernel="stream")
    yt = pw.gemm(x, out_dtype=torch.float32, kernel="tiled")
    torch.cuda.synchronize()
    assert not torch.equal(ys, yt)  # the two kernels sum in different orders: the check can tell them apart
    assert torch.equal(ya, ys if want == "stream" else yt)
    rows = np.arange(0, m, 7)
    ref = O.gemm_ref(prob.x[rows], O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(ya)[rows], ref) <= 1e-4
