"""bench.py end to end on the GPU, at the 32-token workload.

The benchmark is run as its own process (as it is run for the headline
figure) with a short oracle leg, and its JSON line is checked for the fields
every figure is read from: the metric and its value, the roofline of the
dominant kernel, the CPU baseline, the access-pattern ceilings and the
oracle parity verdict on the same outputs.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_tiny_reports_every_field():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--cpu-seconds", "0.5"]
    print("running", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [line for line in res.stdout.splitlines() if line.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "config", "roofline", "cpu_baseline", "ceilings", "parity_ok"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["config"]["workload"].startswith("tiny") or out["config"]["tokens"] == 32
    assert out["value"] is not None and out["value"] > 0
    roof = out["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    base = out["cpu_baseline"]
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0 and base["sample"]
    assert out["parity_checked"] is True and out["parity_ok"] is True
    assert base["parity_max_err_over_bound"] <= 1.0
    route = out["next_subblock_routing"]
    shared = route["shared_component"]
    assert shared["fused_equals_two_kernel"] is True and shared["route_ms"] > 0 and shared["route_fused_ms"] > 0
    assert out["next_consistency"]["fused_route_equals_scores_then_topk"] is True
