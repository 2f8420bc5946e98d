"""Pins of the hard-sample oracle (oracle/sample_oracle.py), on the CPU.

* the Gumbel-max property (a textbook result of the Gumbel-softmax paper in the
  pages' sources): with noise drawn from Gumbel(0, 1), the hard choice of
  kappa * logit + noise is distributed as softmax(kappa * logit);
* a hand-worked 8 x 16 example (tests/golden/hand_sample_8x16.txt);
* tie and NaN rules; every sample is a valid PATCH mask whose sparsity is half
  the fraction of 2:4 tiles;
* planted mistakes (noise subtracted, kappa ignored, patterns reversed, tile
  choice inverted) each fail one of these pins.
"""
import os

import numpy as np
import pytest

import oracle as O
from oracle import sample_oracle as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gumbel(shape, rng):
    u = rng.random(shape)
    return (-np.log(-np.log(u))).astype(np.float32)


def choice_freq(sample_fn, logits, kappa, n=200_000, seed=0):
    rng = np.random.default_rng(seed)
    g = gumbel((n, logits.size), rng)
    idx = sample_fn(np.broadcast_to(logits, g.shape), kappa, g)
    return np.bincount(idx, minlength=logits.size) / n


def oracle_choice(lg, kappa, g):
    return S.first_argmax(S.scores(lg, kappa, g))


def softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("kappa", [1.0, 2.5])
def test_gumbel_max_matches_softmax(kappa):
    logits = np.array([0.3, -0.2, 0.9, 0.0, -1.0, 0.5], np.float32)
    f = choice_freq(oracle_choice, logits, kappa)
    assert np.max(np.abs(f - softmax(kappa * logits.astype(np.float64)))) < 5e-3


def test_planted_noise_sign_and_kappa_fail_the_gumbel_pin():
    logits = np.array([0.3, -0.2, 0.9, 0.0, -1.0, 0.5], np.float32)
    want = softmax(2.5 * logits.astype(np.float64))
    minus = choice_freq(lambda lg, k, g: S.first_argmax(S.scores(lg, k, -g)), logits, 2.5)
    no_kappa = choice_freq(lambda lg, k, g: S.first_argmax(S.scores(lg, 1.0, g)), logits, 2.5)
    assert np.max(np.abs(minus - want)) > 2e-2
    assert np.max(np.abs(no_kappa - want)) > 2e-2


def hand_inputs():
    n, k, tn, tk = 8, 16, 8, 8
    tile_logits = np.array([[0.5, 0.25], [-1.0, 0.5]], np.float32)
    gl = np.zeros((n, k // 4, 6), np.float32)
    for r in range(n):
        for g in range(k // 4):
            gl[r, g, (r + g) % 6] = 1.0
    gl[7, 3, 2] = 1.0  # tie with pattern 4: pattern 2 wins
    return n, k, tn, tk, tile_logits, gl


def read_hand():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "hand_sample_8x16.txt")) if l[0] in "01"]
    return np.array([[int(c) for c in "".join(r)] for r in rows], np.uint8)


def test_hand_worked_example():
    n, k, tn, tk, tl, gl = hand_inputs()
    assert np.array_equal(S.sample_mask(tl, gl, n, k, tn, tk, kappa=2.0), read_hand())


def test_planted_pattern_order_and_tile_inversion_fail_the_hand_example(monkeypatch):
    n, k, tn, tk, tl, gl = hand_inputs()
    monkeypatch.setattr(S, "PATTERNS", tuple(reversed(S.PATTERNS)))
    assert not np.array_equal(S.sample_mask(tl, gl, n, k, tn, tk, 2.0), read_hand())
    monkeypatch.undo()
    assert not np.array_equal(S.sample_mask(tl[:, ::-1].copy(), gl, n, k, tn, tk, 2.0), read_hand())


def test_ties_and_nan():
    s = np.array([[1.0, 1.0, 0.0],            # tie: first wins
                  [np.nan, 0.0, -1.0],         # NaN never wins
                  [np.nan, np.nan, np.nan],    # nothing beats -inf: index 0
                  [-np.inf, -np.inf, -5.0],
                  [np.inf, np.inf, 0.0]], np.float32)
    assert list(S.first_argmax(s)) == [0, 1, 0, 2, 0]


@pytest.mark.parametrize("tn,tk", [(64, 64), (128, 64), (64, 128), (128, 128)])
def test_samples_are_valid_patch_masks(tn, tk):
    rng = np.random.default_rng(tn + tk)
    n, k = 256, 256
    T = (n // tn) * (k // tk)
    tl = rng.normal(0, 0.014, (T, 2)).astype(np.float32)
    gl = rng.normal(0, 0.014, (n, k // 4, 6)).astype(np.float32)
    mask = S.sample_mask(tl, gl, n, k, tn, tk, 25.0, gumbel((T, 2), rng), gumbel((n, k // 4, 6), rng))
    tmap = O.classify(mask, tn, tk)  # raises on an invalid mask
    assert tmap.shape == (T,)
    frac = float(np.mean(tmap == O.SPARSE24))
    assert 0.0 < frac < 1.0
    assert O.measured_sparsity(mask) == pytest.approx(0.5 * frac, abs=1e-12)


def test_one_hot_sample_is_the_magnitude_mask():
    """One-hot tile logits (from a chosen set of 2:4 tiles) and one-hot group logits (the
    magnitude pattern of every group), kappa 1, no noise: the hard sample is exactly the
    generator's magnitude mask of those tiles, written independently in tests/synthetic.py."""
    import synthetic as I
    n, k, tn, tk = 128, 256, 64, 128
    w = I.gen_weight(n, k, I.rng_for(91, 0, I.ROLE_W))
    T = (n // tn) * (k // tk)
    sel = I.choose_sparse_tiles(T, 3, I.rng_for(91, 0, I.ROLE_TILES))
    tl = np.stack([~sel, sel], axis=1).astype(np.float32)
    gl = np.eye(6, dtype=np.float32)[I.magnitude_patterns(w).astype(np.int64)]
    got = S.sample_mask(tl, gl, n, k, tn, tk, 1.0)
    assert np.array_equal(got, I.magnitude_mask(w, sel, tn, tk))
