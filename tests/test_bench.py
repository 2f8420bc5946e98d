"""bench.py host logic (no GPU): the multi-GPU refusal, workload tables and the
weight rotation rule."""
import json
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_workloads_are_whole_tiles_and_named():
    for name in ("llama1b-prefill", "llama7b-decode", "llama7b-prefill", "13b"):
        mats, cfg, desc = bench.workload(name)
        assert mats and desc
        for lbl, m, n, k, (tn, tk), frac in mats:
            assert n % tn == 0 and k % tk == 0 and 0.0 <= frac <= 1.0


def test_nonuniform_layer_hits_the_global_target():
    mats, _, _ = bench.workload("llama7b-prefill")
    tiles = [(n // tn) * (k // tk) for _, _, n, k, (tn, tk), _ in mats]
    sparse = sum(round(f * t) for (*_, f), t in zip(mats, tiles))
    assert sparse == round(0.9 * sum(tiles))


def test_rotation_covers_twice_the_infinity_cache():
    for wb in (16 << 20, 43_000_000, 130_000_000, 600_000_000):
        r = bench.rotation(wb)
        assert r * wb >= 2 * bench.MALL_BYTES and (r - 1) * wb < 2 * bench.MALL_BYTES
    assert 1 <= bench.rotation(0) <= 64
