"""The C ABI from plain C: tests/c_abi_example.c compiles as C11 against
include/lds_gemm.h and links against the library (CPU); on a GPU it runs an
all-ones product (every entry exactly K) and three rejected calls."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lds_staged_matrix_amd")
ROCM = "/opt/rocm"


def _compile(out_dir):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(os.path.join(PKG, "liblds_gemm.so")):
        pytest.skip("library not built")
    exe = os.path.join(out_dir, "c_abi_example")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_example.c"), "-L", PKG, "-llds_gemm",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_compiles_as_c_and_links(tmp_path):
    assert os.path.exists(_compile(str(tmp_path)))


@pytest.mark.gpu
def test_c_program_runs_a_gemm(tmp_path):
    exe = _compile(str(tmp_path))
    print("CASE C ABI example 200x136x264 all ones", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
