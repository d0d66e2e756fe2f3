"""bench.py's one-line JSON report on a small workload: every field the
report promises, with the roofline and CPU-baseline objects."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    print("CASE bench.py --workload bf16_256_nn_f32 --steps 5 --warmup 5", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "bf16_256_nn_f32", "--steps", "5", "--warmup", "5"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert "workload" in d["config"]
    # the clock-settle phase ran before the warm-up steps
    assert d["config"]["settle_steps"] > 0 and d["config"]["settle_ms"] >= 600
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == "TFLOP/s" and cpu["sample"]
