"""Benchmark of the LDS-staged GEMM on one MI355X.

One step = one C <- A*B through the C ABI on the workload's synthetic,
HBM-resident inputs.  The default workload is bf16 M=N=K=8192, A K-contiguous,
B N-contiguous (transposed-LDS-read path), fp32 output.

Prints ONE JSON line on stdout.  Extra per-run detail goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  python bench.py --profile-run      # a few launches only, for rocprofv3
  python bench.py --copy-calibration # one plain 1 GiB device copy, for rocprofv3 --pmc
  python bench.py --variant noswizzle # an A/B build with one design choice changed
  python bench.py --telemetry ...     # the same run as a child process, with socket
                                      # power and GFX clock sampled once a second
"""
import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "bf16 GEMM TFLOP/s + % of MFMA peak; LDS bank-conflict rate (1 MI355X)"
# MI355X dense MFMA peak for bf16/fp16 inputs: 256 CUs x 2.4 GHz x 4096 flop/clk/CU
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12          # 2516.6
# MI355X dense MFMA peak for fp8 inputs: twice the bf16 rate
PEAK_FP8_TFLOPS = 256 * 2.4e9 * 8192 / 1e12           # 5033.2
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_8192_nn_f32"
KERNEL_DIR = "lds_staged_matrix_amd/csrc"
DTYPE_CODE = {("bf16", "f32"): 0, ("bf16", "bf16"): 1, ("f16", "f16"): 2, ("f16", "f32"): 3,
              ("e4m3", "f32"): 4, ("e4m3", "bf16"): 5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text):
    """Source text without comments and blank-line or indentation changes,
    so that editing a comment does not change the kernels' identity."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(l.split()) for l in text.splitlines() if l.strip())


def kernel_source_hash():
    """Identity of the kernel sources that the committed profiles were taken on."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_DIR)
    for name in sorted(os.listdir(d)):
        # the GEMM sources; hw_probe.hip holds test probes, not GEMM kernels
        if name.endswith((".h", ".hip")) and name != "hw_probe.hip":
            h.update(name.encode())
            with open(os.path.join(d, name), encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def read_conflict_rate(workload, layout_name, src_hash):
    """LDS bank-conflict rate (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE) of
    this workload from the committed rocprofv3 counter summary, or None when
    there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "lds_bank_conflicts_all_workloads.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    m = re.search(rf"^rate {re.escape(workload)} {layout_name}:\s*([0-9.eE+-]+)", text, re.M)
    if not m_hash or not m or m_hash.group(1) != src_hash:
        return None
    return float(m.group(1))


def make_inputs(w, layout, inputs="workload"):
    """The workload's seeded operands.  `inputs` = "int" draws integers
    -2..2 instead; "zeros" / "ones" overwrite the device copies with that
    constant (diagnostics of the data-dependent clock only)."""
    import torch
    la, lb = layout
    dist = "int" if inputs == "int" else w["dist"]
    p = synth.make_problem(w["M"], w["N"], w["K"], w["dtype"], la, lb, dist, w["seeds"][0],
                           w["seeds"][1], 1.0 if inputs == "int" else w["scale"])
    raw = (lambda x: x.view(np.int8)) if w["dtype"] == synth.E4M3 else (lambda x: x.view(np.int16))
    A = torch.from_numpy(raw(p.A)).cuda()
    B = torch.from_numpy(raw(p.B)).cuda()
    if inputs in ("zeros", "ones"):
        one = {synth.BF16: 0x3F80, synth.F16: 0x3C00, synth.E4M3: 0x38}[w["dtype"]]
        for t in (A, B):
            t.fill_(0 if inputs == "zeros" else one)
    return p, A, B


def cpu_baseline(p, rows):
    """The oracle, as it is, on `rows` full rows of C of the same problem."""
    import oracle
    ol = {"K": oracle.K_CONTIG, "MN": oracle.MN_CONTIG}
    od = {synth.BF16: oracle.BF16, synth.F16: oracle.F16, synth.E4M3: oracle.E4M3}
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.gemm_rows(p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, ol[p.layoutA], ol[p.layoutB],
                     od[p.dtype], 0, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * p.N * p.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle fp64 m->k->n loop on rows 0..{rows - 1} of the same "
                      f"{p.M}x{p.N}x{p.K} problem ({rows * p.N} outputs), {dt:.2f} s wall"}


def cpu_baseline_all(flop_budget=1.0e10):
    """The oracle, as it stands, timed on this host's cores for every
    workload: configurations small enough for it (256^3, 1500x1152x896) in
    full, one untimed and one timed run, on all cores and on one core; the
    others on their first rows, about `flop_budget` flops' worth, every
    layout.  Prints one JSON line; nothing here touches the GPU."""
    import oracle
    ol = {"K": oracle.K_CONTIG, "MN": oracle.MN_CONTIG}
    od = {synth.BF16: oracle.BF16, synth.F16: oracle.F16, synth.E4M3: oracle.E4M3}
    cores = oracle.max_threads()
    out = {}
    for name, w in synth.WORKLOADS.items():
        full = 2.0 * w["M"] * w["N"] * w["K"] <= 4e9     # 256^3 and 1500x1152x896
        for la, lb in w["layouts"]:
            p = synth.make_problem(w["M"], w["N"], w["K"], w["dtype"], la, lb, w["dist"],
                                   w["seeds"][0], w["seeds"][1], w["scale"])
            rows = p.M if full else max(1, min(p.M, int(flop_budget / (2.0 * p.N * p.K))))

            def run(threads):
                t0 = time.perf_counter()
                oracle.gemm_rows(p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, ol[la], ol[lb],
                                 od[p.dtype], 0, rows, threads=threads)
                return time.perf_counter() - t0
            rec = {"rows": rows, "of_rows": p.M, "cores": cores}
            if full:
                run(0)                                   # untimed
            dt = run(0)
            flops = 2.0 * rows * p.N * p.K
            rec.update(seconds=round(dt, 4), gflops=round(flops / dt / 1e9, 3))
            if full:
                dt1 = run(1)
                rec.update(single_core_seconds=round(dt1, 4),
                           single_core_gflops=round(flops / dt1 / 1e9, 3))
            key = name if len(w["layouts"]) == 1 else f"{name} {la},{lb}"
            out[key] = rec
            log(f"cpu baseline {key}: {rec}")
    print(json.dumps({"cpu_baseline": "oracle fp64 m->k->n loop (OpenMP over m)", "cores": cores,
                      "results": out}), flush=True)


def lds_pad_probe(iters=4096, launches=50, repeats=9):
    """The padding table's measurement ("Lds Optimization", "Optimization
    Method 2: Padding", measured table): one wave reads a strided column of a
    64 x (64 + PAD) fp16 LDS tile, `iters` dependent reads per launch; per PAD
    the best of `repeats` runs of `launches` launches (HIP events on the
    launch stream).  Prints one JSON line: ms per run and the conflict degree
    the bank model predicts (64 banks of 4 bytes, a whole wave per 2-byte
    access)."""
    import ctypes
    import torch
    from lds_staged_matrix_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.HW_PROBE)
    lib.lsm_probe_pad.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lsm_probe_pad.restype = ctypes.c_int
    out = torch.zeros(1, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for pad in (0, 1, 2, 4, 32):
        def launch():
            if lib.lsm_probe_pad(pad, iters, out.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("lsm_probe_pad failed")
        for _ in range(5):
            launch()
        best = None
        for _ in range(repeats):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(launches):
                launch()
            e0.record(stream)
            torch.cuda.synchronize()
            ms = s0.elapsed_time(e0)
            best = ms if best is None else min(best, ms)
        stride_dw = (64 + pad) * 2 / 4.0
        banks = {}
        for t in range(64):
            dw = int((t * (64 + pad) * 2) // 4)
            banks.setdefault(dw % 64, set()).add(dw)
        res[f"pad{pad}"] = {"best_ms_per_run": round(best, 4), "launches_per_run": launches,
                            "reads_per_launch": iters, "row_bytes": 2 * (64 + pad),
                            "model_way": max(len(v) for v in banks.values()),
                            "row_stride_dwords": stride_dw}
        log(f"pad {pad}: best {best:.4f} ms per {launches} launches")
    assert float(out.item()) == 0.0
    print(json.dumps({"probe": "lds padded column read, one wave, 64 x (64 + PAD) fp16",
                      "results": res}), flush=True)



def phase_timeline(workload=HEADLINE, layout=None, launches=100, settle_ms=600.0):
    """Where the ping-pong kernel's cycles go, on a workload that runs it
    (8192^3 by default): the measurement builds `timeline` (the library's
    schedule) and `timeline1` (one loader group) add up, per wave, the
    shader-clock cycles of each phase over the K loop (see LSM_PP_TIMELINE in
    gemm_kernel_pingpong.h).  Each build runs `settle_ms` of launches, then
    `launches` timed ones (HIP events); the counts are those of the last
    launch.  Its C is checked bit for bit against the library's.  Prints the
    table and one JSON line."""
    import ctypes
    import torch
    import lds_staged_matrix_amd as lsm
    from lds_staged_matrix_amd import build as hip_build
    w = synth.WORKLOADS[workload]
    M, N, K = w["M"], w["N"], w["K"]
    layout = tuple(layout.split(",")) if layout else tuple(w["layouts"][0])
    if M % 256 or N % 256 or (M // 256) * (N // 256) < 256:
        sys.exit(f"--phase-timeline: {workload} does not run the ping-pong kernel")
    p, A, B = make_inputs(w, layout)
    gd = DTYPE_CODE[(w["dtype"], w["out"])]
    la = lsm.GEMM_K_CONTIG if layout[0] == "K" else lsm.GEMM_MN_CONTIG
    lb = lsm.GEMM_K_CONTIG if layout[1] == "K" else lsm.GEMM_MN_CONTIG
    stream = torch.cuda.current_stream()
    cdt = torch.float32 if w["out"] == "f32" else torch.int16
    ref = torch.empty(M * N, dtype=cdt, device="cuda")
    h0 = lsm.gemm_create()
    if lsm.gemm_run(h0, A, B, ref, M, N, K, p.lda, p.ldb, N, la, lb, gd, stream) != lsm.GEMM_OK:
        raise RuntimeError("gemm_run failed")
    lsm.gemm_destroy(h0)
    wgs = (M // 256) * (N // 256)
    kt = (K + 63) // 64 if w["dtype"] != synth.E4M3 else (K + 127) // 128
    out = {}
    for name in ("timeline", "timeline1"):
        lib = lsm.ablation_library(name)
        raw = ctypes.CDLL(hip_build.variant_path(name))
        raw.lsm_pp_timeline_set.argtypes = [ctypes.c_void_p]
        raw.lsm_pp_timeline_set.restype = ctypes.c_int
        buf = torch.zeros(wgs * 64, dtype=torch.int64, device="cuda")
        C = torch.empty(M * N, dtype=cdt, device="cuda")
        h = lib.gemm_create()

        def step():
            if lib.gemm_run(h, A, B, C, M, N, K, p.lda, p.ldb, N, la, lb, gd, stream) != lsm.GEMM_OK:
                raise RuntimeError("gemm_run failed")

        if raw.lsm_pp_timeline_set(buf.data_ptr()) != 0:
            raise RuntimeError("lsm_pp_timeline_set failed")
        try:
            t0 = time.perf_counter()
            while (time.perf_counter() - t0) * 1e3 < settle_ms:
                for _ in range(20):
                    step()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(launches):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
        finally:
            raw.lsm_pp_timeline_set(None)
        lib.gemm_destroy(h)
        ms = e0.elapsed_time(e1) / launches
        exact = bool(torch.equal(C, ref))
        t = buf.cpu().numpy().reshape(wgs, 8, 8).astype(np.float64)
        if not (t[:, :, 6] > 0).all():
            raise RuntimeError(f"{name}: a workgroup wrote no counts")
        res = {"ms_per_launch": round(ms, 5), "tflops": round(2.0 * M * N * K / ms / 1e9, 1),
               "equals_library": exact}
        print(f"{name}: {ms:.4f} ms per launch ({res['tflops']} TFLOP/s, HIP events); C equals the library's: {exact}")
        print("  cycles per K tile, mean over workgroups | memory phase | barrier after it | MFMA issue | "
              "wait for own loads | barrier after MFMAs | K loop | prologue (cycles) | epilogue (cycles)")
        for grp, ws in (("group 0", slice(0, 4)), ("group 1", slice(4, 8))):
            v = t[:, ws, :].mean(axis=(0, 1))
            row = [round(x / kt) for x in v[:5]] + [round(v[6] / kt), round(v[5]), round(v[7])]
            res[grp] = row
            print(f"  {grp} | " + " | ".join(str(x) for x in row))
        out[name] = res
        if not exact:
            raise RuntimeError(f"{name}: C differs from the library")
    name = "".join("N" if x == ("K" if i == 0 else "MN") else "T" for i, x in enumerate(layout))
    print(json.dumps({"probe": f"ping-pong phase cycles, {workload} {name}", "results": out}), flush=True)


def lds_read_patterns():
    """(name, mode, 64 lane byte addresses) of the LDS read probe: the
    kernels' own fragment-read addresses (through the host build of
    lds_layout.h) and reference patterns.  Mode 0 ds_read_b64, 1
    ds_read_b64_tr_b8, 2 ds_read_b128."""
    import ctypes
    from lds_staged_matrix_amd import build as hip_build
    lay = ctypes.CDLL(hip_build.layout_host_path(""))
    for f in ("lsm_kc_chunk_offset", "lsm_frag_kc_offset", "lsm_frag16_kc_offset", "lsm_frag_kc8_offset",
              "lsm_frag16_kc8_offset", "lsm_frag_tr8_offset", "lsm_frag16_tr8_offset", "lsm_mn_chunk_offset8"):
        getattr(lay, f).restype = ctypes.c_int
    L = range(64)
    pats = [("linear", 0, [8 * l for l in L]),
            ("linear", 2, [16 * l for l in L]),
            ("kc bf16 32x32 fragment", 2, [lay.lsm_frag_kc_offset(l, 0, 0, 128) for l in L]),
            ("kc bf16 16x16 fragment", 2, [lay.lsm_frag16_kc_offset(l, 0, 0, 128) for l in L]),
            ("kc e4m3 32x32 fragment", 2, [lay.lsm_frag_kc8_offset(l, 0, 0, 0, 128) for l in L]),
            ("kc e4m3 16x16 fragment, chunks g and g+4 (library)", 2,
             [lay.lsm_frag16_kc8_offset(l, 0, 0, 0, 128) for l in L]),
            ("kc e4m3 16x16 fragment, chunks 2g and 2g+1", 2,
             [lay.lsm_kc_chunk_offset(l & 15, 2 * (l >> 4), 128) for l in L]),
            ("tr8 e4m3 32x32 fragment", 1, [lay.lsm_frag_tr8_offset(l, 0, 0, 0, 256) for l in L])]
    for q in range(4):
        pats.append((f"tr8 e4m3 16x16 fragment q{q} (library)", 1,
                     [lay.lsm_frag16_tr8_offset(l, 0, 0, q, 256) for l in L]))
    # the 16x16 reads on the 32x32 fragments' swizzle (rows k and k+16 on one bank)
    pats.append(("tr8 e4m3 16x16 fragment on the 32x32 layout", 1,
                 [lay.lsm_mn_chunk_offset8(16 * (l >> 4) + ((l & 15) >> 1), 0, 256) + 8 * (l & 1) for l in L]))
    return pats


def lds_read_probe(iters=2000, launches=2):
    """One wave repeating one LDS read at given lane addresses
    (libhw_probe.so lsm_probe_lds_read), `launches` launches per pattern in
    the order printed, for counting bank conflicts per pattern with
    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS.
    Prints one JSON line with the patterns, the 4-byte-bank model's degree
    (32-lane phases for 8-byte reads, 16-lane phases for 16-byte reads) and
    the degree of the two-pass model of ds_read_b128."""
    import ctypes
    import torch
    from lds_staged_matrix_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.HW_PROBE)
    lib.lsm_probe_lds_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.lsm_probe_lds_read.restype = ctypes.c_int
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def degree_4b(addrs, width):
        worst, per = 1, 256 // width
        for p0 in range(0, 64, per):
            banks = {}
            for l in range(p0, p0 + per):
                for dw in range(addrs[l] // 4, (addrs[l] + width) // 4):
                    banks.setdefault(dw % 64, set()).add(dw)
            worst = max(worst, max(len(v) for v in banks.values()))
        return worst

    def degree_b128_passes(addrs):
        worst = 1
        for lanes in (list(range(16)) + list(range(32, 48)), list(range(16, 32)) + list(range(48, 64))):
            banks = {}
            for l in lanes:
                banks.setdefault((addrs[l] // 16) % 64, set()).add(addrs[l] // 16)
            worst = max(worst, max(len(v) for v in banks.values()))
        return worst

    rows = []
    for name, mode, addrs in lds_read_patterns():
        arr = (ctypes.c_int * 64)(*addrs)
        for _ in range(launches):
            if lib.lsm_probe_lds_read(mode, arr, iters, out.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError(f"lsm_probe_lds_read refused pattern {name}")
        torch.cuda.synchronize()
        width = 16 if mode == 2 else 8
        rows.append({"pattern": name, "instruction": ["ds_read_b64", "ds_read_b64_tr_b8", "ds_read_b128"][mode],
                     "launches": launches, "reads_per_launch": iters,
                     "model_way_4byte_banks": degree_4b(addrs, width),
                     "model_way_b128_passes": degree_b128_passes(addrs) if mode == 2 else None})
        log(f"lds read probe: {name} ({rows[-1]['instruction']})")
    print(json.dumps({"probe": "lds lane-address reads, one wave", "results": rows}), flush=True)


def parse_amd_smi(text):
    """(socket power in W, GFX_0 clock in MHz) from `amd-smi metric -p -c
    --json` output, or None when the reading has neither."""
    try:
        d = json.loads(text)
        d = d[0] if isinstance(d, list) else d
        if isinstance(d, dict) and "gpu_data" in d:
            d = d["gpu_data"][0]
        val = lambda x: x.get("value") if isinstance(x, dict) else x
        w, c = val(d["power"]["socket_power"]), val(d["clock"]["gfx_0"]["clk"])
        return (float(w), float(c)) if isinstance(w, (int, float)) and isinstance(c, (int, float)) else None
    except (ValueError, KeyError, IndexError, TypeError):
        return None


def summarize_telemetry(samples, loaded_w=600.0):
    """Ranges over the samples taken under load: those above `loaded_w`
    watts, without the first and the last (the clock still moving at the
    start, the load ending during the last second)."""
    loaded = [x for x in samples if x[1] is not None and x[1] > loaded_w][1:-1]
    if not loaded:
        return {"n": 0}
    w = [x[1] for x in loaded]
    c = [x[2] for x in loaded]
    return {"n": len(loaded), "socket_power_w": [min(w), max(w)], "gfx_clk_mhz": [min(c), max(c)],
            "gfx_clk_mhz_mean": round(sum(c) / len(c), 1)}


def run_with_telemetry(argv):
    """Run this benchmark with `argv` as a child process and read amd-smi
    once a second while it runs.  This process itself never touches the GPU.
    Prints the child's JSON line with a `telemetry` object added and returns
    the child's exit status."""
    child = subprocess.Popen([sys.executable, os.path.abspath(__file__)] + argv,
                             stdout=subprocess.PIPE, text=True)
    samples, t0 = [], time.time()
    while child.poll() is None:
        time.sleep(1.0)
        try:
            r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                               text=True, timeout=30)
            reading = parse_amd_smi(r.stdout)
        except (OSError, subprocess.TimeoutExpired):
            reading = None
        samples.append([round(time.time() - t0, 1)] + (list(reading) if reading else [None, None]))
        log(f"telemetry {samples[-1]}")
    out = child.stdout.read()
    lines = [l for l in out.strip().splitlines() if l.startswith("{")]
    if child.returncode != 0 or not lines:
        return child.returncode or 1
    line = json.loads(lines[-1])
    line["telemetry"] = {"source": "amd-smi metric -p -c --json, once a second",
                         "samples_t_s_w_mhz": samples, "loaded": summarize_telemetry(samples)}
    print(json.dumps(line), flush=True)
    return 0


def main():
    if "--telemetry" in sys.argv[1:]:
        sys.exit(run_with_telemetry([a for a in sys.argv[1:] if a != "--telemetry"]))
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 500 untimed and 100 timed launches, the ladder page's test configuration
    # ("An educational GEMM ladder for Helios GPUs", Test Configuration); the
    # chip needs ~80 ms of load before its clock settles.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--settle-ms", type=float, default=600.0,
                    help="before the W warm-up steps, run untimed steps for at least this "
                         "much wall time so the clock has settled under load (0: none)")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--layout", default=None, help="e.g. K,MN (A contiguity, B contiguity)")
    ap.add_argument("--shape", default=None,
                    help="M,N,K: the workload's types, layout and values on another shape "
                         "(a diagnostic line: no traffic or bank-conflict figures)")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="rows of C the oracle computes for the CPU baseline "
                         "(default: about 6e10 flops' worth, 10-20 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--variant", default=None,
                    help="benchmark an A/B build that changes one design choice "
                         "(noswizzle, scalar_tr, ring2, noxcd, stage1, small2, mfma32, poison, waveepi, "
                         "oneloader) instead of the library")
    ap.add_argument("--inputs", default="workload", choices=["workload", "int", "zeros", "ones"],
                    help="operand values: the workload's (default), or integers -2..2, all "
                         "zeros or all ones to show how the clock depends on the data")
    ap.add_argument("--phase-timeline", action="store_true",
                    help="per-phase cycles of the ping-pong kernel at 8192^3 NN (timeline builds), then exit")
    ap.add_argument("--lds-read-probe", action="store_true",
                    help="LDS reads at chosen lane addresses (for the bank-conflict counters), then exit")
    ap.add_argument("--lds-pad-probe", action="store_true",
                    help="time the one-wave strided column read of a 64 x (64 + PAD) fp16 LDS "
                         "tile for PAD 0, 1, 2, 4, 32 (the padding table's probe), for "
                         "calibrating the bank-conflict counters under rocprofv3 --pmc")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="time the oracle on this host for every workload (no GPU use) and exit")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timing of the steps captured in one HIP graph")
    ap.add_argument("--no-flushed", action="store_true",
                    help="skip the 20 launches timed with the caches flushed before each")
    ap.add_argument("--telemetry", action="store_true",
                    help="run the rest of the command as a child process and add amd-smi "
                         "socket power and GFX clock readings, once a second, to its JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this is a single-GPU kernel library "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.cpu_baseline_all:
        cpu_baseline_all()
        return

    import torch
    import lds_staged_matrix_amd as lsm

    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        return

    if args.lds_read_probe:
        lds_read_probe()
        return
    if args.phase_timeline:
        phase_timeline(args.workload, args.layout)
        return
    if args.lds_pad_probe:
        lds_pad_probe()
        return

    w = dict(synth.WORKLOADS[args.workload])
    if args.shape:
        dims = [int(x) for x in args.shape.split(",")]
        if len(dims) != 3 or min(dims) < 1:
            sys.exit("--shape takes M,N,K, three positive sizes")
        w["M"], w["N"], w["K"] = dims
    layout = tuple(args.layout.split(",")) if args.layout else w["layouts"][0]
    gd = DTYPE_CODE[(w["dtype"], w["out"])]
    M, N, K = w["M"], w["N"], w["K"]
    log(f"workload {args.workload} layout {layout} M={M} N={N} K={K}")
    p, A, B = make_inputs(w, layout, args.inputs)
    C = torch.empty(M * N, dtype=torch.float32 if w["out"] == "f32" else torch.int16,
                    device="cuda")
    lib = lsm.ablation_library(args.variant) if args.variant else lsm
    h = lib.gemm_create()
    stream = torch.cuda.current_stream()
    la = lsm.GEMM_K_CONTIG if layout[0] == "K" else lsm.GEMM_MN_CONTIG
    lb = lsm.GEMM_K_CONTIG if layout[1] == "K" else lsm.GEMM_MN_CONTIG

    def step():
        st = lib.gemm_run(h, A, B, C, M, N, K, p.lda, p.ldb, N, la, lb, gd, stream)
        if st != lsm.GEMM_OK:
            raise lsm.GemmError(st, "gemm_run")

    if args.profile_run:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        log("profile run: 5 launches done")
        return

    # Clock settle: under sustained MFMA load the power controller takes
    # tens of milliseconds to bring the clock to its steady level, so a few
    # warm-up steps alone leave the timed steps on a clock that is still
    # moving.  Untimed steps are run, synchronising every 20, until
    # `settle_ms` of wall time have passed; then the W warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` launches back to back; a HIP event pair on
    # the launch stream around every launch gives the kernel's own duration.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    flops = 2.0 * M * N * K
    out_bytes = 4 if w["out"] == "f32" else 2
    in_bytes = 1 if w["dtype"] == synth.E4M3 else 2
    alg_bytes = in_bytes * (M * K + K * N) + out_bytes * M * N
    peak_tflops = PEAK_FP8_TFLOPS if w["dtype"] == synth.E4M3 else PEAK_BF16_TFLOPS
    hbm_bound = flops / alg_bytes < (peak_tflops * 1e12) / (PEAK_HBM_GBS * 1e9)

    # Same kernel with cold caches (the pages' method): before each launch,
    # outside its events, read 1 GiB so that L2 and the 256 MB Infinity Cache
    # hold none of A, B or C.  The flush reads (a write would leave dirty
    # lines whose write-back competes with the timed kernel).
    fl_ms = []
    do_flush = not args.no_flushed
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if do_flush else None
    for i in range(20 if do_flush else 0):
        flush.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        torch.cuda.synchronize()
        fl_ms.append(s.elapsed_time(e))
    del flush

    # The same K steps captured in one HIP graph and replayed: the per-step
    # time without host launch overhead, what a captured loop of GEMMs gets
    # (gemm_run only enqueues kernels, so it can be captured).
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(g, stream=side):
            cs = torch.cuda.current_stream()
            for _ in range(args.steps):
                st = lib.gemm_run(h, A, B, C, M, N, K, p.lda, p.ldb, N, la, lb, gd, cs)
                if st != lsm.GEMM_OK:
                    raise lsm.GemmError(st, "gemm_run (graph capture)")
        stream.wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        g.replay()
        e0.record(stream)
        torch.cuda.synchronize()
        graph_ms = s0.elapsed_time(e0) / args.steps
        del g
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    kavg = float(kern_ms.mean())
    if hbm_bound:
        achieved = alg_bytes / (kavg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / (kavg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": round(peak_tflops, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak_tflops, 4)}
    src_hash = kernel_source_hash()
    roof["traffic"] = read_traffic(args.workload, src_hash) \
        if layout == tuple(w["layouts"][0]) and not args.shape else None

    log(f"kernel ms: mean {kavg:.4f} median {np.median(kern_ms):.4f} min {kern_ms.min():.4f}; "
        f"flushed-cache median {np.median(fl_ms) if fl_ms else float('nan'):.4f} ms; "
        f"wall per step {ms_per_step:.4f} ms; graph replay per step "
        f"{graph_ms if graph_ms is not None else float('nan'):.4f} ms")
    log(f"kernel TFLOP/s {flops / (kavg * 1e-3) / 1e12:.1f}, "
        f"{flops / (kavg * 1e-3) / 1e12 / peak_tflops * 100:.1f}% of the dense "
        f"{'fp8' if in_bytes == 1 else 'bf16'} peak; "
        f"algorithmic GB/s {alg_bytes / (kavg * 1e-3) / 1e9:.1f}")

    cpu = None
    if not args.no_cpu_baseline:
        rows = args.cpu_rows if args.cpu_rows else int(6e10 / (2.0 * N * K))
        rows = max(1, min(rows, M))
        cpu = cpu_baseline(p, rows)
        log(f"cpu baseline: {cpu}")

    unit = "TFLOP/s"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": f"{w['dtype']} GEMM M={M} N={N} K={K}, A "
                               f"{'K' if layout[0] == 'K' else 'M'}-contiguous, B "
                               f"{'K' if layout[1] == 'K' else 'N'}-contiguous, {w['out']} output, "
                               f"fp32 accumulation", "name": args.workload,
                   "M": M, "N": N, "K": K, "layout": "".join("N" if x == ("K" if i == 0 else "MN")
                                                          else "T" for i, x in enumerate(layout)),
                   "inputs": f"{w['dist']} x{w['scale']} seeds {w['seeds']}" if args.inputs == "workload"
                             else f"{args.inputs} (diagnostic, not the workload's values)",
                   "kernel_ms_mean": round(kavg, 5), "kernel_ms_flushed_median":
                       round(float(np.median(fl_ms)), 5) if fl_ms else None,
                   "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
                   "kernel_source_hash": src_hash,
                   "settle_steps": settle_steps, "settle_ms": round(settle_ms, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    line["config"]["lds_bank_conflict_rate"] = None if args.variant or args.shape else \
        read_conflict_rate(args.workload, line["config"]["layout"], src_hash)
    if args.shape:
        line["config"]["name"] = f"{args.workload} at {M}x{N}x{K}"
    if args.variant:
        line["config"]["ablation_build"] = args.variant
        roof["traffic"] = None
    lib.gemm_destroy(h)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
