"""GPU parity of the hard tile-configuration sample (patch_sample_mask) against
the oracle (oracle/sample_oracle.py): the mask bits must be equal bit for bit,
both sides deciding every argmax in fp32 with the same rounding.  Logits are
drawn like the card's initialisation (N(0, 0.014)) and larger, Gumbel noise is
an input, kappa spans the card's schedule (25 -> 350)."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import sample_oracle as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def gumbel(shape, rng):
    return (-np.log(-np.log(rng.random(shape)))).astype(np.float32)


def inputs(n, k, tn, tk, seed, scale=0.014, noise=True):
    rng = np.random.default_rng(seed)
    T = (n // tn) * (k // tk)
    tl = rng.normal(0, scale, (T, 2)).astype(np.float32)
    gl = rng.normal(0, scale, (n, k // 4, 6)).astype(np.float32)
    tz = gumbel((T, 2), rng) if noise else None
    gz = gumbel((n, k // 4, 6), rng) if noise else None
    return tl, gl, tz, gz


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(P, n, k, tn, tk, kappa, tl, gl, tz, gz, order="big"):
    bits = P.sample_mask(dev(tl), dev(gl), n, k, tile=(tn, tk), kappa=kappa, tile_noise=dev(tz),
                         group_noise=dev(gz), bit_order=order)
    torch.cuda.synchronize()
    want = S.sample_mask(tl, gl, n, k, tn, tk, kappa, tz, gz)
    return bits.cpu().numpy(), np.packbits(want.reshape(-1), bitorder=order), want


@pytest.mark.parametrize("tn,tk", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("kappa", [25.0, 350.0])
def test_bits_equal_the_oracle(P, tn, tk, kappa):
    n, k = 384, 512
    tl, gl, tz, gz = inputs(n, k, tn, tk, seed=tn * 3 + tk + int(kappa))
    got, want, _ = run(P, n, k, tn, tk, kappa, tl, gl, tz, gz)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("order", ["big", "little"])
def test_bit_orders_and_no_noise(P, order):
    n, k, tn, tk = 256, 256, 64, 64
    tl, gl, _, _ = inputs(n, k, tn, tk, seed=81, scale=1.0, noise=False)
    got, want, _ = run(P, n, k, tn, tk, 1.0, tl, gl, None, None, order)
    assert np.array_equal(got, want)


def test_ties_nan_and_inf(P):
    n, k, tn, tk = 128, 128, 64, 64
    tl, gl, tz, gz = inputs(n, k, tn, tk, seed=82, scale=1.0)
    rng = np.random.default_rng(83)
    gz[:] = 0.0
    gl[:] = np.round(gl * 2) / 2          # many exact ties among the six scores
    flat = gl.reshape(-1)
    for v in (np.nan, np.inf, -np.inf):
        flat[rng.choice(flat.size, 500, replace=False)] = v
    gl[3, 5, :] = np.nan                   # a group with nothing but NaN: pattern 0
    tl[0] = [np.nan, 1.0]                  # NaN dense score: 2:4 wins
    tl[1] = [1.0, 1.0]                     # tie: dense wins
    tz[:] = 0.0
    got, want, mask = run(P, n, k, tn, tk, 25.0, tl, gl, tz, gz)
    assert np.array_equal(got, want)
    assert mask[3, 20:24].tolist() == [1, 1, 0, 0]  # tile 0 is 2:4; the all-NaN group takes pattern (0,1)
    assert O.classify(mask, tn, tk)[1] == O.DENSE   # tied tile scores: dense


def test_sample_packs_into_the_sampled_tile_types(P):
    n, k, tn, tk = 512, 1024, 128, 128
    tl, gl, tz, gz = inputs(n, k, tn, tk, seed=84)
    bits = P.sample_mask(dev(tl), dev(gl), n, k, tile=(tn, tk), kappa=100.0, tile_noise=dev(tz),
                         group_noise=dev(gz))
    w = torch.randn((n, k), device="cuda").to(torch.bfloat16)
    pw = P.pack(w, bits, tile=(tn, tk))
    want_types = S.first_argmax(S.scores(tl, 100.0, tz))
    assert np.array_equal(pw.export()["tile_map"], want_types.astype(np.uint8))


def test_argument_errors(P):
    tl, gl, _, _ = inputs(128, 128, 64, 64, seed=85)
    with pytest.raises(ValueError):
        P.sample_mask(dev(tl), dev(gl)[:, :16], 128, 128, tile=(64, 64))
    with pytest.raises(P.PatchError) as e:
        P.sample_mask(dev(np.zeros((8, 2), np.float32)), dev(gl), 128, 128, tile=(64, 32))
    assert e.value.status_name == "PATCH_E_SHAPE"


@pytest.mark.parametrize("tn,tk", [(128, 128), (64, 128)])
def test_one_hot_sample_is_the_magnitude_mask(P, tn, tk):
    """The configuration the model-stack benchmark uses to build its masks: one-hot tile
    logits from a chosen set of 2:4 tiles, one-hot group logits from the magnitude
    pattern of every group, kappa 1, no noise.  The bits equal the host generator's
    magnitude mask of the same tiles, bit for bit."""
    import synthetic as I
    n, k = 512, 1024
    w = I.gen_weight(n, k, I.rng_for(90, 0, I.ROLE_W))
    T = (n // tn) * (k // tk)
    sel = I.choose_sparse_tiles(T, int(0.7 * T), I.rng_for(90, 0, I.ROLE_TILES))
    tl = np.stack([~sel, sel], axis=1).astype(np.float32)
    gl = np.eye(6, dtype=np.float32)[I.magnitude_patterns(w).astype(np.int64)]
    bits = P.sample_mask(dev(tl), dev(gl), n, k, tile=(tn, tk), kappa=1.0).cpu().numpy()
    want = I.pack_mask_bits(I.magnitude_mask(w, sel, tn, tk))
    assert np.array_equal(bits, want)
