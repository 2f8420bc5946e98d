"""GPU parity at the largest weight the library accepts: N * K just below
PATCH_MAX_WEIGHTS (2^31 - 1), where the GEMM kernels' 32-bit pool offsets
come closest to their limit.

The 46336 x 46336 weight (2 147 024 896 weights, 362 x 362 tiles of 128 x 128)
is generated on the device with a seeded torch generator: W ~ N(0, 0.02) in
bf16, each tile dense with probability 0.9 (so that the dense pool, 3.9 GB,
reaches offsets past 2^31 bytes) and otherwise 2:4 with one of the six keep
patterns per group of four along K, chosen at random (any valid PATCH mask
will do here; the magnitude reading is not needed).  Checked:
  * the tile counts against the mask's own;
  * unpack of the first and last tile rows against W times the keep mask,
    bit for bit;
  * Y on sampled output columns (the first and last W rows, whose tiles sit
    at the lowest and highest pool offsets) against the fp64 oracle, for the
    streaming kernel (M = 16) and the 256-row tiled kernel (M = 256).
About 16 GB of device memory at the peak; skipped when less than 32 GB is free.
"""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

N = K = 46336          # 362 * 128; N * K = 2 147 024 896 <= 2^31 - 1
TN = TK = 128
TOL = 1e-2
PATTERNS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 32 * 2**30:
        pytest.skip("needs 32 GB of free device memory")
    from sparse_gemm_patch_amd import api
    api.load()
    assert N * K <= 2**31 - 1 and N % TN == 0 and K % TK == 0
    g = torch.Generator(device="cuda")
    g.manual_seed(0x50415443)
    w = (torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    tiles_n, tiles_k = N // TN, K // TK
    sparse_tile = torch.rand((tiles_n, tiles_k), generator=g, device="cuda") >= 0.9
    pat = torch.zeros((6, 4), dtype=torch.uint8, device="cuda")
    for i, (a, b) in enumerate(PATTERNS):
        pat[i, a] = pat[i, b] = 1
    pidx = torch.randint(0, 6, (N, K // 4), generator=g, device="cuda", dtype=torch.uint8)
    keep = pat[pidx.long().view(-1)].view(N, K)  # 2:4 everywhere, then dense tiles set to all ones
    del pidx
    dense_rows = (~sparse_tile).repeat_interleave(TN, 0).repeat_interleave(TK, 1)
    keep[dense_rows] = 1
    del dense_rows
    weights = torch.tensor([128, 64, 32, 16, 8, 4, 2, 1], dtype=torch.uint8, device="cuda")
    bits = torch.empty(N * K // 8, dtype=torch.uint8, device="cuda")
    chunk = 1 << 26  # bytes of bits per pass, bounding the temporaries
    kv = keep.view(-1, 8)
    for s in range(0, bits.numel(), chunk):
        e = min(s + chunk, bits.numel())
        bits[s:e] = (kv[s:e] * weights).sum(dim=1, dtype=torch.int32).to(torch.uint8)
    del kv
    pw = api.pack(w, bits, tile=(TN, TK))
    torch.cuda.synchronize()
    yield api, w, keep, sparse_tile, pw
    del pw, w, keep, bits
    torch.cuda.empty_cache()


def test_max_size_tile_counts(big):
    api, w, keep, sparse_tile, pw = big
    n_sparse = int(sparse_tile.sum().item())
    assert pw.info["n_sparse"] == n_sparse
    assert pw.info["n_dense"] == sparse_tile.numel() - n_sparse
    # the dense pool reaches past 2^31 bytes, so its last tiles sit at offsets that a signed 32-bit
    # offset could not hold
    assert pw.info["bytes_dense"] > 2**31


def test_max_size_unpack_first_and_last_tile_rows(big):
    api, w, keep, sparse_tile, pw = big
    wm = pw.unpack()
    torch.cuda.synchronize()
    for r0 in (0, N - TN):
        want = torch.where(keep[r0:r0 + TN].bool(), w[r0:r0 + TN], torch.zeros((), dtype=w.dtype, device="cuda"))
        assert torch.equal(wm[r0:r0 + TN].view(torch.int16), want.view(torch.int16)), r0
    del wm


@pytest.mark.parametrize("m,kernel", [(16, "stream"), (256, "tiled")])
def test_max_size_gemm_sampled_columns(big, m, kernel):
    api, w, keep, sparse_tile, pw = big
    g = torch.Generator(device="cuda")
    g.manual_seed(0x50415443 + m)
    x = torch.randn((m, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = pw.gemm(x, kernel=kernel, block_m=256 if kernel == "tiled" else 0)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(0, 4), np.arange(N - 68, N - 64), np.arange(N - 4, N),
                                     np.random.default_rng(m).choice(N, size=8, replace=False)]))
    ci = torch.from_numpy(cols).cuda()
    x_bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    w_rows = w[ci].view(torch.int16).cpu().numpy().view(np.uint16)
    k_rows = keep[ci].cpu().numpy().astype(np.uint8)
    ref = O.gemm_ref(x_bits, O.masked_weight(w_rows, k_rows))
    got = y[:, ci].float().cpu().numpy().astype(np.float64)
    assert O.rel_error(got, ref) <= TOL
