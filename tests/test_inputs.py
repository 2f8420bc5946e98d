"""Input generators (no GPU): the per-group pattern form of the magnitude 2:4
mask equals the mask form, ties included."""
import numpy as np

import synthetic as I

PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def test_magnitude_patterns_match_magnitude_mask():
    rng = np.random.default_rng(0)
    w = I.gen_weight(64, 256, rng)
    w[0, :4] = w[0, 0]          # four equal magnitudes: positions 0 and 1 kept
    w[1, 4:8] = [w[1, 4], w[1, 4] ^ 0x8000, 0, 0]  # equal magnitudes of opposite sign
    pat = I.magnitude_patterns(w)
    mask = I.magnitude_mask(w, np.ones(4, bool), 64, 64)
    rebuilt = np.zeros((64, 64, 4), np.uint8)
    for p, (a, b) in enumerate(PAIRS):
        rebuilt[..., a][pat == p] = 1
        rebuilt[..., b][pat == p] = 1
    assert np.array_equal(rebuilt.reshape(64, 256), mask)
    assert pat[0, 0] == 0 and pat[1, 1] == 0
