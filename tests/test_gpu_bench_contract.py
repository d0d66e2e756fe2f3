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
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == "TFLOP/s" and cpu["sample"]


@pytest.mark.parametrize("workload,output", [("f16_1500x1152x896_nn_f16", "f16"),
                                             ("e4m3_8192_nn_f32", "bf16")])
def test_bench_vs_hipblaslt_reports_both_sides(workload, output):
    """The hipBLASLt reference point: both sides timed on the same operands."""
    print(f"CASE bench.py --workload {workload} --vs-hipblaslt --steps 3 --warmup 3", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload,
                        "--steps", "3", "--warmup", "3", "--no-cpu-baseline", "--no-graph",
                        "--no-flushed", "--vs-hipblaslt"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    v = d["config"]["vs_hipblaslt"]
    assert v is not None and v["output"] == output
    for side in ("hipblaslt", "library", "hipblaslt_again"):
        assert v[side + "_ms"] > 0 and v[side + "_tflops"] > 0
    if workload.startswith("e4m3"):
        assert v["layout"] == "NT"
