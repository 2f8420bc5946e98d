"""Seeded synthetic inputs for the hybrid dense / 2:4 tile GEMM.

Test and measurement infrastructure: the CPU oracle's tests, the GPU parity
tests, the smoke check and the benchmark draw their inputs from here; the
library never imports it.  It draws random numbers and builds masks; it holds
none of the packing or GEMM arithmetic that the library and the oracle
implement.

The workloads follow the PATCH pages:
  * weights are an ``nn.Linear`` weight ``W[N][K]`` (out x in), loaded in bf16
    (model card "llama_3.2_1b-PATCH-45Sparse", section "How to use");
  * the released artifact is a binary keep/prune mask, bit-packed
    (same card, description);
  * each tile of W is dense or 2:4 sparse, and the global sparsity is set by
    the fraction of 2:4 tiles (same card, description; "PATCH: Learnable
    Tile-level Hybrid Sparsity for LLMs", Abstract);
  * tile sizes 128x128, 128x64, 64x128 and 64x64
    (card, "Training hyper-parameters", mask tile size row).

The real masks and weights are not available, so synthetic stand-ins are
drawn: W ~ N(0, 0.02), X ~ N(0, 1), rounded to bf16 (round to nearest even);
2:4 tiles keep the two largest |w| of every aligned group of four along K
(the magnitude criterion, used here only to generate masks), ties going to
the lower index; sparse tiles are a uniform random subset of the tiles.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 0x50415443  # "PATC"
ROLE_W, ROLE_X, ROLE_TILES, ROLE_FRACTIONS, ROLE_LOGITS = 0, 1, 2, 3, 4


def rng_for(cfg: int, matrix: int, role: int) -> np.random.Generator:
    """PCG64 generator for one (config, matrix, role) triple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, cfg, matrix, role])))


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    NaN inputs are not expected (the generators draw finite normals)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- tensors

def gen_weight(n: int, k: int, rng: np.random.Generator, sigma: float = 0.02) -> np.ndarray:
    """W[n][k] as bf16 bits, W ~ N(0, sigma)."""
    return f32_to_bf16_bits(rng.normal(0.0, sigma, size=(n, k)).astype(np.float32))


def gen_x(m: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """X[m][k] as bf16 bits, X ~ N(0, 1)."""
    return f32_to_bf16_bits(rng.standard_normal(size=(m, k)).astype(np.float32))


# ---------------------------------------------------------------- tile choice

def sparse_tile_count(frac: float, tiles: int) -> int:
    """Number of 2:4 tiles for a target fraction: floor(frac*tiles + 0.5)."""
    return int(math.floor(frac * tiles + 0.5))


def choose_sparse_tiles(tiles: int, n_sparse: int, rng: np.random.Generator) -> np.ndarray:
    """Boolean[tiles]: a uniform random subset of n_sparse tiles (row-major tile order)."""
    if not 0 <= n_sparse <= tiles:
        raise ValueError("n_sparse out of range")
    sel = np.zeros(tiles, dtype=bool)
    sel[rng.permutation(tiles)[:n_sparse]] = True
    return sel


def magnitude_top2(w_bits: np.ndarray) -> np.ndarray:
    """u8[N][K]: 1 where a weight is one of the two largest |w| of its aligned group of four
    along K (on equal magnitudes the lower index wins)."""
    n, k = w_bits.shape
    mag = np.abs(bf16_bits_to_f32(w_bits)).reshape(n, k // 4, 4)
    # stable argsort on -|w| keeps the lower index first among equal magnitudes
    order = np.argsort(-mag, axis=2, kind="stable")
    top2 = np.zeros_like(mag, dtype=np.uint8)
    np.put_along_axis(top2, order[:, :, :2], 1, axis=2)
    return top2.reshape(n, k)


def hybrid_mask(top2: np.ndarray, tile_sparse: np.ndarray, tn: int, tk: int) -> np.ndarray:
    """Keep mask u8[N][K]: the 2:4 pattern `top2` inside the 2:4 tiles, all ones elsewhere.
    ``tile_sparse`` is Boolean[(N/tn)*(K/tk)] in row-major tile order."""
    n, k = top2.shape
    sp = np.asarray(tile_sparse, dtype=bool).reshape(n // tn, k // tk)
    elem_sparse = np.repeat(np.repeat(sp, tn, axis=0), tk, axis=1)
    return np.where(elem_sparse, top2, np.uint8(1)).astype(np.uint8)


def magnitude_mask(w_bits: np.ndarray, tile_sparse: np.ndarray, tn: int, tk: int) -> np.ndarray:
    """Keep/prune mask u8[N][K] (1 = keep).

    Dense tiles keep everything.  In a 2:4 tile every aligned group of four
    along K keeps its two largest |w|; on equal magnitudes the lower index wins.
    ``tile_sparse`` is Boolean[(N/tn)*(K/tk)] in row-major tile order."""
    return hybrid_mask(magnitude_top2(w_bits), tile_sparse, tn, tk)


# Code i0 | i1 << 2 of a 2:4 group -> index of its pattern in the order
# (0,1) (0,2) (0,3) (1,2) (1,3) (2,3).
_PATTERN_OF_CODE = {4: 0, 8: 1, 12: 2, 9: 3, 13: 4, 14: 5}


def magnitude_patterns(w_bits: np.ndarray) -> np.ndarray:
    """int8[N][K/4]: per aligned group of four along K, the index of the 2:4 pattern that keeps
    its two largest |w| (lower index first among equal magnitudes, as magnitude_mask)."""
    n, k = w_bits.shape
    mag = np.abs(bf16_bits_to_f32(w_bits)).reshape(n, k // 4, 4)
    order = np.sort(np.argsort(-mag, axis=2, kind="stable")[:, :, :2], axis=2)
    code = order[:, :, 0] | (order[:, :, 1] << 2)
    lut = np.zeros(16, np.int8)
    for c, p in _PATTERN_OF_CODE.items():
        lut[c] = p
    return lut[code]


def pack_mask_bits(mask: np.ndarray, order: str = "big") -> np.ndarray:
    """Bit-pack a 0/1 mask, flattened row-major, with numpy.packbits ('big' = MSB first)."""
    return np.packbits(np.asarray(mask, dtype=np.uint8).reshape(-1), bitorder=order)


# ---------------------------------------------------------------- workloads

@dataclass
class Problem:
    """One synthetic hybrid-tile GEMM problem (all arrays are host numpy)."""
    name: str
    m: int
    n: int
    k: int
    tn: int
    tk: int
    w: np.ndarray          # uint16 [n][k] bf16 bits
    x: np.ndarray          # uint16 [m][k] bf16 bits
    mask: np.ndarray       # uint8  [n][k] 0/1
    bits: np.ndarray       # uint8  packed mask, MSB first
    tile_sparse: np.ndarray  # bool [T]
    meta: dict = field(default_factory=dict)


def make_problem(name: str, m: int, n: int, k: int, tn: int, tk: int, frac: float | None = None,
                 n_sparse: int | None = None, cfg: int = 0, matrix: int = 0,
                 order: str = "big") -> Problem:
    """Seeded problem: W, X, a random subset of 2:4 tiles, the magnitude mask and its bits."""
    if n % tn or k % tk:
        raise ValueError("shape not divisible by tile")
    tiles = (n // tn) * (k // tk)
    if n_sparse is None:
        n_sparse = sparse_tile_count(0.0 if frac is None else frac, tiles)
    w = gen_weight(n, k, rng_for(cfg, matrix, ROLE_W))
    x = gen_x(m, k, rng_for(cfg, matrix, ROLE_X))
    sel = choose_sparse_tiles(tiles, n_sparse, rng_for(cfg, matrix, ROLE_TILES))
    mask = magnitude_mask(w, sel, tn, tk)
    bits = pack_mask_bits(mask, order)
    return Problem(name, m, n, k, tn, tk, w, x, mask, bits, sel, {"n_sparse": n_sparse, "tiles": tiles})


# Llama-3.2-1B linears (out x in)
LLAMA32_1B = {"q": (2048, 2048), "k": (512, 2048), "v": (512, 2048), "o": (2048, 2048),
              "gate": (8192, 2048), "up": (8192, 2048), "down": (2048, 8192)}
# LLaMA-2-7B linears
LLAMA2_7B = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
             "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
# 13B-shaped linears
LLAMA2_13B = {"qkvo": (5120, 5120), "gate_up": (13824, 5120), "down": (5120, 13824)}


def nonuniform_fractions(tile_counts: list[int], rng: np.random.Generator, lo: float = 0.3,
                         hi: float = 1.0, global_frac: float = 0.9) -> tuple[np.ndarray, list[int]]:
    """Per-matrix 2:4-tile counts with fractions drawn from U[lo, hi], shifted by one common
    offset (bisection) so that the total is round(global_frac * sum(tiles)).

    Returns (fractions, sparse tile counts).  Leftover tiles after flooring go to the
    largest fractional parts, ties to the lower matrix index."""
    t = np.asarray(tile_counts, dtype=np.float64)
    u = rng.uniform(lo, hi, size=len(tile_counts))
    target = global_frac * t.sum()
    a, b = -1.0, 1.0
    for _ in range(200):
        c = 0.5 * (a + b)
        if (t * np.clip(u + c, lo, hi)).sum() < target:
            a = c
        else:
            b = c
    f = np.clip(u + 0.5 * (a + b), lo, hi)
    s = np.floor(t * f).astype(np.int64)
    want = int(math.floor(target + 0.5))
    rem = want - int(s.sum())
    frac_part = t * f - s
    order = sorted(range(len(s)), key=lambda i: (-frac_part[i], i))
    for i in order[:max(rem, 0)]:
        s[i] += 1
    return f, [int(v) for v in s]


def sample_inputs(n: int, k: int, tn: int, tk: int, rng: np.random.Generator, scale: float = 0.014,
                  noise: bool = True):
    """Seeded inputs of a hard tile-configuration sample: tile logits [T][2], group logits
    [n][k/4][6] ~ N(0, scale) (the card's logit initialisation is N(0, 0.014)), and standard
    Gumbel noise of the same shapes, -log(-log(u)) with u uniform in (0, 1), all float32."""
    tiles = (n // tn) * (k // tk)
    tl = rng.normal(0.0, scale, (tiles, 2)).astype(np.float32)
    gl = rng.normal(0.0, scale, (n, k // 4, 6)).astype(np.float32)
    if not noise:
        return tl, gl, None, None
    u = rng.random((tiles, 2))
    tz = (-np.log(-np.log(u))).astype(np.float32)
    u = rng.random((n, k // 4, 6))
    gz = (-np.log(-np.log(u))).astype(np.float32)
    return tl, gl, tz, gz
