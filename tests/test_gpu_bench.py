"""bench.py end to end on the GPU: every op that the benchmark runs prints
one JSON line with the keys of its contract (a few steps each, no CPU
baseline, smallest buffer rotation).  bench.py runs as a child process, as
it does for a user; this process holds no GPU memory while it runs."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "cpu_baseline"}


@pytest.mark.parametrize("op", ["glu", "add_rmsnorm", "glu_strided", "gemm_glu", "mlp", "configs"])
def test_bench_op_prints_its_line(op):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--op", op, "--steps", "5", "--warmup", "2",
           "--sets", "2", "--no-cpu-baseline", "--no-torch-eager"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=180, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    out = json.loads(lines[0])
    assert KEYS <= set(out), sorted(KEYS - set(out))
    assert out["n_gpus"] == 1 and out["value"] and out["value"] > 0
    assert "workload" in out["config"]
    if op == "configs":
        assert len(out["rows"]) == 21 and all(r["fwd_GBps"] > 0 and r["bwd_GBps"] > 0 for r in out["rows"])
    elif op != "mlp":
        roof = out["roofline"]
        assert roof["peak"] > 0 and 0 < roof["frac"] < 1 and roof["bound"] in ("hbm", "mfma")
    if op in ("glu", "glu_strided", "add_rmsnorm"):
        # the same-run ceiling from the data-movement reference kernels
        assert 0 < out["pct_of_attainable"] < 120
        attain = {"glu": lambda a: a["bwd_mix"]["GBps"], "add_rmsnorm": lambda a: a["GBps"],
                  "glu_strided": lambda a: a["tile_bwd_mix"]["GBps"]}[op](out["attainable"])
        assert 0 < attain < 8000


def test_bench_gemm_shape_sweep():
    """--gemm-shapes adds the fused / unfused comparison over other MLP shapes
    and the path GatedMLP's default takes for each."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--op", "gemm_glu", "--gemm-shapes", "--steps", "5",
           "--warmup", "2", "--no-cpu-baseline"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    sweep = out["shape_sweep"]
    assert len(sweep) == 25
    for row in sweep:
        assert row["fused_us"] > 0 and row["unfused_us"] > 0
        tiles = -(-row["M"] // 128) * -(-row["intermediate"] // 64)
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        assert row["auto_picks_fused"] == (row["M"] <= 256 and tiles <= ncu)

