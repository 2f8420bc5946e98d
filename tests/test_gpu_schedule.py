"""GPU tests of the launch schedule (cost prefix, cost-ordered groups, ragged-round
tails of 256-row blocks run as 192-row blocks in the same launch).

Block heights change which workgroup computes an output, never the order of its
K sum, so a tail-split launch must equal the uniform 256-row launch bit for bit;
both are also checked against the oracle on sampled rows."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I
from conftest import ROOT

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


def rows_of(m, seed, count=24):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=count, replace=False)]))


# (M, N, K, tile, 2:4 fraction): each leaves a ragged last round of 256 x 256 blocks on
# 256 workgroups (19 x 16 = 304 blocks; 43 x 16 = 688; 54 x 8 = 432)
SPLIT = [(4096, 4864, 512, (128, 128), 0.9), (4096, 11008, 4096, (128, 128), 0.9),
         (2048, 13824, 5120, (128, 64), 0.9)]


@pytest.mark.parametrize("m,n,k,tile,frac", SPLIT, ids=[f"{s[1]}x{s[2]}-M{s[0]}" for s in SPLIT])
def test_tail_split_equals_uniform_blocks(P, m, n, k, tile, frac):
    prob = I.make_problem("tail", m, n, k, tile[0], tile[1], frac=frac, cfg=80, matrix=n % 13)
    pw = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=tile)
    x = dev_u16(prob.x)
    auto = pw.gemm(x)                                    # library plan (tail split)
    uniform = pw.gemm(x, kernel="tiled", block_m=256)    # forced height: no split
    torch.cuda.synchronize()
    assert torch.equal(auto, uniform)
    rows = rows_of(m, n)
    got = auto[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    ref = O.gemm_ref(prob.x[rows], O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(got, ref) <= TOL


PLAN_SCRIPT = r"""
import json, sys
import numpy as np, torch
sys.path[:0] = [{root!r}, {tests!r}]
import synthetic as I
from sparse_gemm_patch_amd import api
m, n, k, tn, tk, frac = {args!r}
prob = I.make_problem("plan", m, n, k, tn, tk, frac=frac, cfg=81)
d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
pw = api.pack(d(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(tn, tk))
pw.gemm(d(prob.x))
torch.cuda.synchronize()
print("done", flush=True)
"""


def launch_plan(args):
    code = PLAN_SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"), args=tuple(args))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, PATCH_LOG="1"), cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return [ln for ln in r.stderr.splitlines() if ln.startswith("patch: k_gemm_tiled")]


def test_tail_split_is_planned():
    """The 11008 x 4096 product at M = 4096 (2.69 rounds of 256-row blocks): 32 block
    columns stay at 256 rows (512 blocks, two rounds), the other 11 run as 192-row
    blocks (11 x 22 = 242) in the same launch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lines = launch_plan((4096, 11008, 256, 128, 128, 0.9))
    assert len(lines) == 1, lines
    entries = lines[0].split("|")[1:]
    assert len(entries) == 2, lines[0]
    assert "rows 0..8192" in entries[0] and "bm 256 blocks 512" in entries[0]
    assert "rows 8192..11008" in entries[1] and "bm 192 blocks 242" in entries[1]


def test_whole_rounds_are_not_split():
    """8192 x 2048 at M = 4096 fills exactly two rounds: one entry, no tail."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lines = launch_plan((4096, 8192, 256, 128, 128, 0.9))
    assert len(lines) == 1 and lines[0].count("|") == 1, lines


def test_clustered_dense_rows_cost_order(P):
    """A group whose products differ in their dense / 2:4 mix (all dense, half, all 2:4 by
    tile rows) is dispatched most expensive first; every product still equals its solo
    launch bit for bit and the oracle on sampled rows."""
    probs = []
    for i, frac in enumerate([1.0, 0.5, 0.0]):
        probs.append(I.make_problem("mix", 1024, 2560, 1024, 128, 128, frac=frac, cfg=82, matrix=i))
    pws = [P.pack(dev_u16(p.w), torch.from_numpy(p.bits).cuda(), tile=(128, 128)) for p in probs]
    xs = [dev_u16(p.x) for p in probs]
    ys = P.gemm_grouped(list(zip(pws, xs)))
    solo = [pw.gemm(x) for pw, x in zip(pws, xs)]
    torch.cuda.synchronize()
    for p, y, s in zip(probs, ys, solo):
        assert torch.equal(y, s)
        rows = rows_of(p.m, 7)
        got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        assert O.rel_error(got, O.gemm_ref(p.x[rows], O.masked_weight(p.w, p.mask))) <= TOL
