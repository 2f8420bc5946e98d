"""GPU parity over seeded random shapes: every tile size, ragged M, strided X and Y,
random sparsity and output type, the library's own kernel choice and a forced one.

Each case checks the packed format bit for bit against the oracle, Y against the
fp64 oracle (all rows up to 300, 64 sampled rows above), bf16 Y against fp32 Y
rounded to nearest even, and, for prefill-sized M, bitwise equality of Y across
block heights (every kernel accumulates K in the same order), and the call with a
workspace: against the oracle where it splits K, bitwise equal to the call
without one where it does not."""
import os

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu

TILES = [(128, 128), (128, 64), (64, 128), (64, 64)]
CASES = int(os.environ.get("PATCH_RANDOM_CASES", "32"))  # more for a longer sweep


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def case(i):
    rng = np.random.default_rng([0x5241, i])
    tn, tk = TILES[rng.integers(len(TILES))]
    n = tn * int(rng.integers(1, 13))
    k = tk * int(rng.integers(1, 25))
    m = int(rng.choice([rng.integers(1, 17), rng.integers(17, 301), rng.integers(1000, 3001)]))
    frac = float(rng.choice([0.0, 1.0, rng.random()]))
    pad_x = 8 * int(rng.integers(0, 3))
    pad_y = 8 * int(rng.integers(0, 3))
    f32 = bool(rng.integers(2))
    if rng.random() < 0.25:  # a wide weight: 2 or 4 W blocks per streaming workgroup
        n = tn * int(rng.integers(5120 // tn, 12288 // tn + 1))
    if rng.random() < 0.1:  # a narrow weight with a long K at m <= 128: the K split over a workspace
        n = tn * int(rng.integers(2048 // tn, 5119 // tn + 1))
        k = tk * int(rng.integers(8192 // tk, 12288 // tk + 1))
        m = int(rng.integers(1, 129))
    return dict(tn=tn, tk=tk, n=n, k=k, m=m, frac=frac, pad_x=pad_x, pad_y=pad_y, f32=f32)


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(P, i):
    c = case(i)
    print(f"case {i}: {c}", flush=True)
    prob = I.make_problem("rnd", c["m"], c["n"], c["k"], c["tn"], c["tk"], frac=c["frac"], cfg=200, matrix=i)
    pw = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(c["tn"], c["tk"]))
    ref_pack = O.compress(prob.w, prob.mask, c["tn"], c["tk"])
    got = pw.export()
    for key in ("tile_map", "tile_slot", "dense_vals", "sparse_vals", "sparse_meta"):
        assert np.array_equal(got[key], getattr(ref_pack, key)), key

    xs = torch.zeros((c["m"], c["k"] + c["pad_x"]), dtype=torch.bfloat16, device="cuda")
    xs[:, :c["k"]] = dev_u16(prob.x)
    x = xs[:, :c["k"]]
    dt = torch.float32 if c["f32"] else torch.bfloat16
    ys = torch.full((c["m"], c["n"] + c["pad_y"]), float("nan"), dtype=dt, device="cuda")
    y = ys[:, :c["n"]]
    pw.gemm(x, out=y, out_dtype=dt)
    y32 = pw.gemm(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    if c["pad_y"]:
        assert torch.isnan(ys[:, c["n"]:]).all()  # nothing written past n
    if c["f32"]:
        assert torch.equal(y, y32)
    else:
        assert torch.equal(y, y32.to(torch.bfloat16))

    rows = np.arange(c["m"]) if c["m"] <= 300 else np.sort(np.random.default_rng(i).choice(c["m"], 64, replace=False))
    ref = O.gemm_ref(prob.x[rows], O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y32.cpu().numpy().astype(np.float64)[rows], ref) <= 1e-4

    # AUTO ran one of the two kernels: streaming for m <= 16, the tiled kernel past 128 rows,
    # either in between (its cost estimate decides); every forced form is checked as well
    yt = pw.gemm(x, out_dtype=torch.float32, kernel="tiled") if c["m"] > 16 else None
    ys_ = pw.gemm(x, out_dtype=torch.float32, kernel="stream") if c["m"] <= 128 else None
    torch.cuda.synchronize()
    if yt is not None:
        for bm in (256, 192, 128, 64):
            yb = pw.gemm(x, out_dtype=torch.float32, kernel="tiled", block_m=bm)
            torch.cuda.synchronize()
            assert torch.equal(yb, yt), bm
    if ys_ is not None:
        assert O.rel_error(ys_.cpu().numpy().astype(np.float64)[rows], ref) <= 1e-4
    if c["m"] <= 16:
        assert torch.equal(ys_, y32)
    elif c["m"] > 128:
        assert torch.equal(yt, y32)
    else:
        assert torch.equal(ys_, y32) or torch.equal(yt, y32)

    # with a workspace (filled with NaN: stale contents must not matter) the library may split K
    need = pw.workspace_size(c["m"])
    ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")
    yw = pw.gemm(x, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    if need == 0:
        assert torch.equal(yw, y32)  # nothing to split: the launch without a workspace
    else:
        assert O.rel_error(yw.cpu().numpy().astype(np.float64)[rows], ref) <= 1e-4
