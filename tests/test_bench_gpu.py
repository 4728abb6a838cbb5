"""bench.py end to end on the GPU, headline only: one JSON line on stdout with
the fields the benchmark contract names, and a roofline that follows from
its own numbers."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_quick_bench_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py --quick --steps 3 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--quick", "--steps", "3", "--warmup", "1"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["dtype"] == "bf16" and j["higher_is_better"] is True
    assert j["config"]["workload"].startswith("dense_8k_bf16")
    roof = j["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert 0.0 < roof["frac"] < 1.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    # achieved = algorithmic FLOPs per launch / average launch time
    assert roof["achieved"] == pytest.approx(roof["flop_per_launch"] / (roof["avg_launch_ms"] * 1e-3) / 1e12,
                                             rel=2e-3)
    assert j["value"] > 0 and j["ms_per_step"] > 0
