"""GPU tests of the grouped launch (patch_gemm_grouped): several linears of a
layer in one launch per kernel.

Each product of a group must equal, bit for bit, the same product run alone
through patch_gemm, and the oracle within the GEMM tolerance.  Groups mix tile
shapes, K, ragged M, decode-sized M (streaming kernel) with prefill-sized M
(tiled kernel), shared and separate X, and products with nothing to do."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def packed(P, prob):
    return P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(prob.tn, prob.tk))


def y_host(y):
    return y.float().cpu().numpy().astype(np.float64)


def run_group(P, probs, out_dtype, kernel="auto", block_m=0, shared_x=False):
    """Grouped result vs solo results (bitwise) and vs the oracle."""
    pws = [packed(P, p) for p in probs]
    xs = [dev_u16(p.x) for p in probs]
    if shared_x:
        xs = [xs[0]] * len(xs)
    ys = P.gemm_grouped(list(zip(pws, xs)), out_dtype=out_dtype, kernel=kernel, block_m=block_m)
    solo = [pw.gemm(x, out_dtype=out_dtype, kernel=kernel, block_m=block_m) for pw, x in zip(pws, xs)]
    torch.cuda.synchronize()
    for i, (p, y, s) in enumerate(zip(probs, ys, solo)):
        assert torch.equal(y, s), f"product {i} differs from its solo launch"
        xp = probs[0].x if shared_x else p.x
        ref = O.gemm_ref(xp, O.masked_weight(p.w, p.mask))
        err = O.rel_error(y_host(y), ref)
        assert err <= (1e-4 if out_dtype == torch.float32 else TOL), (i, err)
    return ys


def layer(m, cfg, scale=4, fracs=(0.9,) * 7):
    """The seven LLaMA-3.2-1B projections with their dimensions divided by `scale`."""
    probs = []
    for i, (lbl, (n, k)) in enumerate(I.LLAMA32_1B.items()):
        probs.append(I.make_problem(lbl, m, n // scale, k // scale, 128, 128, frac=fracs[i], cfg=cfg, matrix=i))
    return probs


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m", [1, 16, 300])
def test_layer_group_equals_solo(P, m, out_dtype):
    """q, k, v, o, gate, up, down (K = 512 and 2048 mixed) in one group."""
    run_group(P, layer(m, cfg=60, fracs=(0.9, 0.5, 0.7, 0.9, 1.0, 0.0, 0.9)), out_dtype)


def test_shared_x_group(P):
    """q, k, v on one X, as a fused QKV would run them."""
    probs = layer(257, cfg=61)[:3]
    for p in probs[1:]:
        assert p.k == probs[0].k
    run_group(P, probs, torch.bfloat16, shared_x=True)


@pytest.mark.parametrize("block_m", [256, 192, 128, 64])
def test_group_forced_block_rows(P, block_m):
    probs = layer(200, cfg=62)
    run_group(P, probs, torch.float32, kernel="tiled", block_m=block_m)


def test_group_forced_stream(P):
    probs = [I.make_problem("s", m, 256, k, 128, 64, frac=0.5, cfg=63, matrix=j)
             for j, (m, k) in enumerate([(1, 64), (5, 192), (16, 1088), (3, 2048)])]
    run_group(P, probs, torch.float32, kernel="stream")


def test_mixed_tiles_and_sizes(P):
    """Every tile shape, decode and prefill M, ragged M and N in one group."""
    specs = [(1, 384, 640, 128, 128, 0.5), (300, 640, 1024, 64, 64, 0.9), (17, 256, 512, 128, 64, 0.0),
             (16, 512, 256, 64, 128, 1.0), (130, 128, 128, 128, 128, 1.0), (1000, 256, 384, 64, 128, 0.3)]
    probs = [I.make_problem("mx", m, n, k, tn, tk, frac=f, cfg=64, matrix=j)
             for j, (m, n, k, tn, tk, f) in enumerate(specs)]
    run_group(P, probs, torch.bfloat16)
    run_group(P, probs, torch.float32)


def test_sixteen_products(P):
    probs = [I.make_problem("g16", 33 + 29 * j, 128 * (1 + j % 3), 128 * (1 + j % 4), 64, 64,
                            frac=(j % 5) / 4, cfg=65, matrix=j) for j in range(16)]
    run_group(P, probs, torch.float32)


def test_group_with_empty_products(P):
    """m = 0 and K = 0 items in a group: skipped / all-zero Y, the others unaffected."""
    probs = layer(40, cfg=66)[:2]
    pws = [packed(P, p) for p in probs]
    w0 = torch.zeros((128, 0), dtype=torch.bfloat16, device="cuda")
    pw_k0 = P.pack(w0, torch.zeros(1, dtype=torch.uint8, device="cuda"), tile=(64, 64))
    x_k0 = torch.zeros((9, 0), dtype=torch.bfloat16, device="cuda")
    x_m0 = torch.zeros((0, probs[1].k), dtype=torch.bfloat16, device="cuda")
    items = [(pws[0], dev_u16(probs[0].x)), (pw_k0, x_k0), (pws[1], x_m0), (pws[1], dev_u16(probs[1].x))]
    ys = P.gemm_grouped(items, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], pws[0].gemm(items[0][1], out_dtype=torch.float32))
    assert tuple(ys[1].shape) == (9, 128) and bool(torch.all(ys[1] == 0))
    assert tuple(ys[2].shape) == (0, probs[1].n)
    assert torch.equal(ys[3], pws[1].gemm(items[3][1], out_dtype=torch.float32))


def test_empty_group_is_noop(P):
    assert P.gemm_grouped([]) == []


def test_group_errors_launch_nothing(P):
    """A bad item is named and no product of the group is computed."""
    probs = layer(24, cfg=67)[:3]
    pws = [packed(P, p) for p in probs]
    xs = [dev_u16(p.x) for p in probs]
    outs = [torch.full((24, p.n), 7.0, dtype=torch.float32, device="cuda") for p in probs]
    wide = torch.zeros((24, probs[2].k + 8), dtype=torch.bfloat16, device="cuda")
    lib = P.load()
    items = (P.GemmItem * 3)()
    for i in range(3):
        items[i] = P.GemmItem(pws[i]._h, xs[i].data_ptr(), 24, probs[i].k, outs[i].data_ptr(), probs[i].n)
    items[2].x = wide.data_ptr() + 2  # misaligned X in the third product
    st = lib.patch_gemm_grouped(items, 3, 1, None)
    assert P.STATUS[st] == "PATCH_E_INVALID_ARG"
    assert "product 2" in lib.patch_last_error().decode()
    torch.cuda.synchronize()
    for o in outs:
        assert bool(torch.all(o == 7.0))
    with pytest.raises(ValueError):
        P.gemm_grouped([(pws[0], xs[0])] * 17)
    big = (P.GemmItem * 17)()
    for i in range(17):
        big[i] = items[0]
    st = lib.patch_gemm_grouped(big, 17, 1, None)
    assert P.STATUS[st] == "PATCH_E_INVALID_ARG"
    over = (P.GemmItem * 2)(items[0], items[1])
    over[1].m = 129  # forced streaming past its 128 rows: rejected before any launch
    st = lib.patch_gemm_grouped_kernel(over, 2, 1, 2, 0, None)
    assert P.STATUS[st] == "PATCH_E_INVALID_ARG"
    assert "product 1" in lib.patch_last_error().decode()


def test_block_rows_do_not_change_bits(P):
    """The tiled kernel's block height changes which workgroup computes an
    element, not the order of its sum: a group may pick another height than a
    solo launch and still match it bit for bit."""
    prob = I.make_problem("bmbits", 300, 640, 1024, 128, 128, frac=0.6, cfg=68)
    pw = packed(P, prob)
    x = dev_u16(prob.x)
    ys = [pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=b) for b in (256, 192, 128, 64)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kernel", ["auto", "stream"])
def test_group_mixing_stream_batch_sizes(P, kernel, out_dtype):
    """Streamed items of 4, 40 and 100 rows (1, 4 and 8 blocks of 16 X rows per wave; the first with
    16 waves, the others with 8 in a launch of their own) beside a tiled one: each equals its solo
    launch bit for bit."""
    specs = [(4, 512, 4096, 128, 128, 0.9), (40, 256, 4096, 128, 64, 0.5), (100, 256, 8192, 64, 128, 0.7)]
    if kernel == "auto":
        specs.append((300, 512, 512, 128, 128, 0.9))
    probs = [I.make_problem("mix", m, n, k, tn, tk, frac=f, cfg=71, matrix=i)
             for i, (m, n, k, tn, tk, f) in enumerate(specs)]
    run_group(P, probs, out_dtype, kernel=kernel)


@pytest.mark.parametrize("kernel", ["auto", "stream"])
def test_group_mixing_stream_families(P, kernel):
    """Streamed items whose wave counts and W blocks per workgroup differ (one W block with 16 or 8
    waves, 2 and 4 W blocks with 8) run in one launch per family; each equals its solo launch bit
    for bit and the oracle."""
    specs = [(8, 10240, 320, 64, 64, 0.9), (40, 5120, 256, 128, 128, 0.5), (20, 1024, 512, 128, 64, 0.7),
             (100, 10240, 384, 128, 128, 0.3), (50, 512, 384, 64, 128, 1.0), (3, 5120, 128, 64, 64, 0.0),
             (128, 256, 640, 128, 128, 0.6)]
    probs = [I.make_problem("fam", m, n, k, tn, tk, frac=f, cfg=72, matrix=i)
             for i, (m, n, k, tn, tk, f) in enumerate(specs)]
    run_group(P, probs, torch.float32, kernel=kernel)
    run_group(P, probs, torch.bfloat16, kernel=kernel)
