"""Wait-state rules around the inline-assembly direct-to-LDS loads, checked on
the built gfx950 code objects (CPU only: the libraries are disassembled, not run).

The kernels issue `buffer_load_dwordx4 ... lds` from inline assembly, and the
compiler's hazard recognizer does not look inside asm statements, so the two
gfx9-family wait-state rules that apply to these loads are the source's job:
  * a scalar write of M0 needs one wait state before an LDS-DMA load reads M0
    (the compiler emits `s_nop 0` there for its own buffer-load-to-LDS builtin);
  * a VALU instruction that writes an SGPR needs five wait states before a
    vector memory instruction reads that SGPR.
Every LDS-DMA load of every built kernel library is checked against both.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lds_staged_matrix_amd")
LLVM = "/opt/rocm/llvm/bin"
BUNDLER = os.path.join(LLVM, "clang-offload-bundler")
OBJDUMP = os.path.join(LLVM, "llvm-objdump")


def _libraries():
    libs = [os.path.join(PKG, "liblds_gemm.so")]
    abl = os.path.join(PKG, "ablation")
    if os.path.isdir(abl):
        libs += sorted(os.path.join(abl, f) for f in os.listdir(abl) if f.endswith(".so"))
    return [p for p in libs if os.path.exists(p)]


def _disassemble(lib, tmp_path):
    """Instruction texts of the gfx950 code object embedded in `lib`."""
    fat = tmp_path / "fat.bin"
    co = tmp_path / "co.o"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib, str(fat)],
                   check=True)
    subprocess.run([BUNDLER, "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], check=True,
                         capture_output=True, text=True).stdout
    ins = []
    for line in out.splitlines():
        if not line.startswith("\t"):
            if line.endswith(">:"):
                ins.append(None)                 # function start: no hazard crosses it
            continue
        text = line.split("//")[0].strip()
        if text:
            ins.append(text)
    return ins


def _sgprs(operand):
    regs = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", operand):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[])s(\d+)\b", operand):
        regs.add(int(m.group(1)))
    return regs


def _wait_states(text):
    m = re.match(r"s_nop\s+(?:0x)?([0-9a-f]+)", text)
    return int(m.group(1), 16 if "0x" in text else 10) + 1 if m else 1


def _scalar_dest(text):
    """SGPRs written by a VALU instruction (readfirstlane, readlane, compares
    to an SGPR pair, carry-out forms); empty for everything else."""
    if not text.startswith("v_"):
        return set()
    ops = text.split(None, 1)[1] if " " in text else ""
    first = ops.split(",")[0].strip()
    return _sgprs(first) if first.startswith("s") else set()


needs_tools = pytest.mark.skipif(
    not (os.path.exists(BUNDLER) and os.path.exists(OBJDUMP) and shutil.which("objcopy")),
    reason="ROCm LLVM tools or objcopy not present")


@needs_tools
@pytest.mark.parametrize("lib", _libraries() or [None],
                         ids=lambda p: os.path.basename(p) if p else "unbuilt")
def test_lds_dma_wait_states(lib, tmp_path):
    if lib is None:
        pytest.skip("kernel library not built")
    ins = _disassemble(lib, tmp_path)
    loads = [i for i, t in enumerate(ins) if t and t.startswith("buffer_load") and t.endswith(" lds")]
    assert loads, "no direct-to-LDS loads found"
    for i in loads:
        ops = [o.strip() for o in ins[i].split(None, 1)[1].split(",")]
        read = set().union(*(_sgprs(o) for o in ops[1:]))
        waits = 0
        for j in range(i - 1, max(i - 8, -1), -1):
            prev = ins[j]
            if prev is None:
                break
            if re.match(r"s_\w+\s+m0\b", prev):
                assert waits >= 1, f"{os.path.basename(lib)}: M0 written right before {ins[i]!r}"
            if waits < 5:
                assert not (_scalar_dest(prev) & read), \
                    f"{os.path.basename(lib)}: {prev!r} feeds {ins[i]!r} after {waits} wait states"
            waits += _wait_states(prev)


def test_scalar_dest_parser():
    assert _scalar_dest("v_readfirstlane_b32 s4, v1") == {4}
    assert _scalar_dest("v_cmp_gt_i32_e64 s[8:9], s3, v2") == {8, 9}
    assert _scalar_dest("v_add_u32_e32 v1, s2, v3") == set()
    assert _scalar_dest("s_mov_b32 m0, s3") == set()
    assert _wait_states("s_nop 0") == 1 and _wait_states("s_nop 4") == 5
    assert _wait_states("v_mov_b32_e32 v1, v2") == 1
