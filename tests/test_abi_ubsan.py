"""gemm_run's argument validation under the undefined-behaviour sanitizer.

The library source (host code instrumented with -fsanitize=undefined, every
report fatal) is linked with tests/abi_validation_driver.cpp, which runs each
request of the ABI validation table in test_abi.py through gemm_run on the
CPU.  The statuses must match the table, and no request may reach undefined
behaviour: sizes whose byte footprints approach 2^63, leading dimensions up
to 2^40 and the fp8 32-bit offset check all stay within int64 arithmetic.
(A build of the earlier validation code, whose offset check multiplied
without an overflow test, fails here with a signed-overflow report.)
No GPU is used: requests that pass validation stop at the device check.
"""
import os
import subprocess

import pytest

from lds_staged_matrix_amd import build as hip_build
from test_abi import VALIDATION_CASES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(hip_build.HIPCC):
        pytest.skip("hipcc is not available")
    out = str(tmp_path_factory.mktemp("ubsan") / "abi_validation")
    # -O1: the kernels' inline-assembly loads need their scalar operands in SGPRs
    cmd = [hip_build.HIPCC, "-O1", "--offload-arch=gfx950", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", hip_build.CSRC,
           os.path.join(hip_build.CSRC, "gemm_api.hip"),
           os.path.join(ROOT, "tests", "abi_validation_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_validation_table_without_undefined_behaviour(driver):
    lines = "".join(" ".join(str(int(x)) for x in args) + "\n" for args, _ in VALIDATION_CASES)
    r = subprocess.run([driver], input=lines, capture_output=True, text=True, timeout=120)
    assert "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stderr[-3000:]
    got = [int(x) for x in r.stdout.split()]
    want = [status for _, status in VALIDATION_CASES]
    assert got == want
