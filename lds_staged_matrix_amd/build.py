"""Build the HIP library liblds_gemm.so in-tree with hipcc for gfx950.

Also builds, from the same sources:
  * ablation/liblds_gemm_<name>.so -- the A/B builds that each change one
    design choice (see VARIANTS), used by the benchmark and the counter runs
    that measure what each choice buys;
  * liblds_layout_host.so (and _noswizzle) -- host-only builds of the LDS
    address functions, evaluated by the bank-conflict model in the tests;
  * libhw_probe.so -- one-wave probe kernels of the hardware behaviour the
    kernels rely on (fragment reads, MFMA layouts, buffer range checks, padded
    LDS column reads), for the tests and the benchmark's probe mode.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblds_gemm.so")
ABLATION_DIR = os.path.join(PKG, "ablation")
SOURCES = ["gemm_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
         # keep packed fp32 instructions out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]

# One design choice changed per build; the library itself uses none of these.
VARIANTS = {
    "noswizzle": ["-DLSM_LDS_SWIZZLE=0"],   # row-major LDS tiles, no XOR swizzle
    "scalar_tr": ["-DLSM_TR_READ=0"],       # 8 x 16-bit LDS reads instead of ds_read_b64_tr_b16
    "ring2": ["-DLSM_RING_STAGES=2"],       # M <= 32 kernel with a 2-stage instead of 6-stage ring
    "noxcd": ["-DLSM_XCD_REMAP=0"],         # tiles in hardware workgroup order, not grouped per XCD
    "stage1": ["-DLSM_DMA_STAGES=1"],       # 128/64 direct-to-LDS kernel with one LDS stage, no overlap
    "small2": ["-DLSM_SMALL_FOUR_STAGES=0"],  # 64 x 64 tile always double-buffered, never four stages
    "mfma32": ["-DLSM_PP_MFMA=32", "-DLSM_PP_MFMA8=32"],   # ping-pong kernel on 32x32 MFMAs (32x32x16, fp8 32x32x64)
    "poison": ["-DLSM_LDS_POISON=1"],       # LDS filled with NaN bits before each region's first use
    # C staged per wave (ping-pong, 128 x 128 tile) or stored from the accumulators (64 x 64 tile)
    # instead of staged for the whole workgroup
    "waveepi": ["-DLSM_PP_ROW_EPI=0", "-DLSM_DMA_ROW_EPI=0"],
    "oneloader": ["-DLSM_PP_SPLIT_LOADS=0"],  # ping-pong: group 0 issues every load, for every layout (no split, 2 B stages)
    # measurement builds: the ping-pong kernel counts its phase cycles (bench.py --phase-timeline)
    "timeline": ["-DLSM_PP_TIMELINE=1"],
    "timeline1": ["-DLSM_PP_TIMELINE=1", "-DLSM_PP_SPLIT_LOADS=0"],
}

LAYOUT_HOST = {"": [], "_noswizzle": ["-DLSM_LDS_SWIZZLE=0"]}
HW_PROBE = os.path.join(PKG, "libhw_probe.so")


def variant_path(name: str) -> str:
    return os.path.join(ABLATION_DIR, f"liblds_gemm_{name}.so")


def layout_host_path(suffix: str = "") -> str:
    return os.path.join(PKG, f"liblds_layout_host{suffix}.so")


def _run(cmd, out, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l)   # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, extra_flags=(), variant: str = None) -> str:
    """Build the library (or, with `variant`, one ablation build)."""
    out = LIB
    flags = list(extra_flags)
    if variant is not None:
        os.makedirs(ABLATION_DIR, exist_ok=True)
        out = variant_path(variant)
        flags = VARIANTS[variant] + flags
    cmd = [HIPCC, *FLAGS, *flags, "-shared",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    return _run(cmd, out, verbose)


def build_hw_probe(verbose: bool = False) -> str:
    """The probe kernels (device code, same flags as the library)."""
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "hw_probe.hip"), "-o", HW_PROBE + ".tmp"]
    return _run(cmd, HW_PROBE, verbose)


def build_layout_host(verbose: bool = False):
    """Host-only builds of the LDS address functions (no device code)."""
    outs = []
    for suffix, flags in LAYOUT_HOST.items():
        out = layout_host_path(suffix)
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", "-x", "hip", "--offload-host-only",
               "-I", CSRC, *flags, os.path.join(CSRC, "layout_probe.cpp"), "-o", out + ".tmp"]
        outs.append(_run(cmd, out, verbose))
    return outs


def build_all(verbose: bool = False):
    """Every build, six hipcc processes at a time."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [lambda: build(verbose)] + [lambda n=n: build(verbose, variant=n) for n in VARIANTS] + \
           [lambda: build_layout_host(verbose), lambda: build_hw_probe(verbose)]
    with ThreadPoolExecutor(max_workers=6) as pool:
        for f in [pool.submit(j) for j in jobs]:
            f.result()


if __name__ == "__main__":
    build_all(verbose=True)
