"""bench.py end to end on the GPU: one JSON line with the fields the benchmark
contract names, a roofline whose fraction is its achieved rate over its peak, and
a CPU-oracle baseline that also checked the GPU output.  Runs the default
(1B prefill) and the decode workload with few steps, each in a child process."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

TOP = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
       "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")


def run_bench(*extra, sweep=False):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           *([] if sweep else ["--no-sweep"]), "--no-grouped", "--no-sample", "--no-split", *extra]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(d, steps=3, warmup=1):
    for key in TOP:
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert isinstance(d["config"], dict) and d["config"]["workload"]
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    return r


def test_default_workload_line():
    d = run_bench("--cpu-rows", "256")
    r = check_common(d)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    # value is the dense-equivalent rate of the step
    assert abs(d["dense_equiv_frac_of_peak"] - d["value"] / 2500.0) < 1e-3
    c = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in c, key
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["parity_max_rel"] <= 1e-2


def test_decode_workload_line():
    d = run_bench("--workload", "llama7b-decode", "--no-cpu-baseline", sweep=True)
    r = check_common(d)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert d["cpu_baseline"] is None and d["weight_copies"] >= 2
    assert sorted(d["other_m"]) == ["M=1", "M=128", "M=32", "M=64", "M=8"]
    assert all(v["dense_eq_tflops"] > 0 for v in d["other_m"].values())
    # every decode batch size at every sparsity: 3 shapes x 3 M x 3 sparsities
    g = d["decode_grid"]
    assert sorted(g) == ["M=1", "M=16", "M=8"]
    assert all(len(row) == 3 and all(v["dense_eq_tflops"] > 0 for v in row.values()) for row in g.values())
    assert g["M=16"] and sorted(g["M=16"]) == sorted(d["sweep"])


@pytest.mark.parametrize("wl", ["llama7b-model-prefill", "llama7b-model-decode"])
def test_model_stack_line(wl):
    """The whole-model linear stack, two layers: the line's contract, and the first
    layer's products checked against the oracle on a row sample."""
    d = run_bench("--workload", wl, "--layers", "2", "--cpu-rows", "64")
    r = check_common(d)
    assert d["config"]["layers"] == 2
    assert r["bound"] == ("mfma" if wl.endswith("prefill") else "hbm")
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["parity_max_rel"] <= 1e-2
    assert d["grouped"]["ms_per_step"] > 0
