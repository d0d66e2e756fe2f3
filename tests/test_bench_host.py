"""Host-side logic of bench.py (no GPU): the one-GPU guard, the readers of the
committed rocprofv3 summaries, and the oracle CPU-baseline leg."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert h == bench.kernel_source_hash()


def _recorded_hash(name):
    text = open(os.path.join(ROOT, "profiles", name)).read()
    return re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M).group(1)


@pytest.mark.parametrize("workload", ["bf16_8192_nn_f32", "e4m3_8192_nn_f32",
                                      "bf16_skinny_32x16384x8192_nn_bf16"])
def test_traffic_is_read_only_for_the_profiled_sources(workload):
    rec = _recorded_hash(f"hbm_traffic_{workload}.txt")
    got = bench.read_traffic(workload, rec)
    assert got is not None and got > 0
    assert bench.read_traffic(workload, "0" * 16) is None
    assert bench.read_traffic("no_such_workload", rec) is None


def test_conflict_rate_is_read_only_for_the_profiled_sources():
    rec = _recorded_hash("lds_bank_conflicts_all_workloads.txt")
    for wl, lay in [("bf16_8192_nn_f32", "NN"), ("bf16_4096_all_bf16", "NT")]:
        v = bench.read_conflict_rate(wl, lay, rec)
        assert v is not None and 0.0 <= v < 0.05
        assert bench.read_conflict_rate(wl, lay, "0" * 16) is None


def test_cpu_baseline_times_the_oracle_on_a_sample():
    p = synth.make_problem(48, 40, 32, synth.BF16, "K", "MN", "uniform", 1, 2)
    r = bench.cpu_baseline(p, 8)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "rows 0..7" in r["sample"]


def test_lds_read_probe_patterns_are_in_range_and_aligned():
    # bench.py --lds-read-probe hands these to the probe kernel, whose host
    # entry refuses anything outside its 64 KiB LDS or misaligned; every
    # pattern must pass that check, and every mode must be one it knows
    pats = bench.lds_read_patterns()
    assert len({(n, m) for n, m, _ in pats}) == len(pats)
    for name, mode, addrs in pats:
        width = 16 if mode == 2 else 8
        assert mode in (0, 1, 2) and len(addrs) == 64, name
        assert all(0 <= a and a % width == 0 and a + width <= 65536 for a in addrs), name


def test_lds_read_probe_patterns_cover_the_measured_cases():
    # the profile's table pins the two-pass form of ds_read_b128 with the
    # kernels' own fragment reads and the one pattern that tells the models
    # apart (chunks 2g, 2g + 1 of 16 consecutive 128-byte rows)
    names = {n for n, _, _ in bench.lds_read_patterns()}
    assert "kc e4m3 16x16 fragment, chunks 2g and 2g+1" in names
    assert "kc e4m3 16x16 fragment, chunks g and g+4 (library)" in names
    text = open(os.path.join(ROOT, "profiles", "lds_bank_passes_read_probe.txt")).read()
    for n in names:
        assert n in text, n


def test_amd_smi_reading_is_parsed_from_its_json_forms():
    one = {"power": {"socket_power": {"value": 1398, "unit": "W"}},
           "clock": {"gfx_0": {"clk": {"value": 1805, "unit": "MHz"}}}}
    assert bench.parse_amd_smi(json.dumps(one)) == (1398.0, 1805.0)
    assert bench.parse_amd_smi(json.dumps([one])) == (1398.0, 1805.0)
    assert bench.parse_amd_smi(json.dumps({"gpu_data": [one]})) == (1398.0, 1805.0)
    plain = {"power": {"socket_power": 700}, "clock": {"gfx_0": {"clk": 2400}}}
    assert bench.parse_amd_smi(json.dumps(plain)) == (700.0, 2400.0)
    assert bench.parse_amd_smi("") is None
    assert bench.parse_amd_smi(json.dumps({"power": {"socket_power": "N/A"},
                                           "clock": {"gfx_0": {"clk": 2400}}})) is None


def test_telemetry_ranges_keep_the_loaded_samples_only():
    samples = [[1.0, 300.0, 2100.0], [2.0, 1300.0, 2000.0], [3.0, 1398.0, 1810.0],
               [4.0, 1400.0, 1790.0], [5.0, None, None], [6.0, 1390.0, 1800.0], [7.0, 900.0, 2300.0],
               [8.0, 250.0, 2100.0]]
    s = bench.summarize_telemetry(samples)
    # above 600 W: t = 2, 3, 4, 6, 7; the first and the last of those are dropped
    assert s["n"] == 3
    assert s["socket_power_w"] == [1390.0, 1400.0]
    assert s["gfx_clk_mhz"] == [1790.0, 1810.0]
    assert bench.summarize_telemetry([[1.0, 100.0, 2000.0]]) == {"n": 0}


def test_telemetry_run_passes_the_child_status_through():
    # the child refuses more than one GPU before touching any; no JSON line
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--telemetry", "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
