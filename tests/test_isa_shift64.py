"""The built library's own gfx950 code, disassembled: no 64-bit shift takes its shift amount from
a VGPR.

On MI355X a v_lshlrev_b64 whose shift amount sat in the last VGPR of an 8-register allocation
block (v15 in the 2:4 unpack) now and then shifted by a wrong amount: in the full-size
round-trip tests, every one of 283 wrong dense groups was reproduced exactly by the two such
shifts of that kernel taking another amount, and by nothing else.  The kernels place values and
index fields with 32-bit operations instead; this test keeps any variable-amount 64-bit shift
out of the library, whatever the register allocation does.  (Shifts by an immediate, as in
address arithmetic, are not affected and are allowed.)

The code object is extracted from libnm_mask.so (its .hip_fatbin section), unbundled for gfx950
and disassembled with the ROCm LLVM tools; no GPU is needed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "semi_structured_sparsity_amd", "libnm_mask.so")
LLVM = "/opt/rocm/llvm/bin"
SHIFT64 = re.compile(r"^\s*(v_lshlrev_b64|v_lshrrev_b64|v_ashrrev_i64)(_e64)?\s+v\[\d+:\d+\],\s*([^,\s]+)")


def _disassemble(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libnm_mask.so is not built")
    tools = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"), os.path.join(LLVM, "llvm-objdump")]
    if not all(t and os.path.exists(t) for t in tools):
        pytest.skip("objcopy / clang-offload-bundler / llvm-objdump not available")
    objcopy, bundler, objdump = tools
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fat)], check=True)
    targets = subprocess.run([bundler, "--list", "--type=o", f"--input={fat}"], check=True, capture_output=True,
                             text=True).stdout.split()
    gfx = [t for t in targets if t.endswith("gfx950")]
    assert gfx, f"no gfx950 code object in {LIB}: {targets}"
    co = tmp_path / "co.o"
    subprocess.run([bundler, "--unbundle", "--type=o", f"--input={fat}", f"--targets={gfx[0]}", f"--output={co}"],
                   check=True)
    return subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True, capture_output=True,
                          text=True).stdout


def shift64_by_register(disassembly):
    """[(function, instruction)] for every 64-bit shift whose amount operand is a VGPR."""
    found, fn = [], None
    for line in disassembly.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:", line)
        if m:
            fn = m.group(1)
            continue
        m = SHIFT64.match(line)
        if m and re.fullmatch(r"v\d+", m.group(3)):
            found.append((fn, line.split("//")[0].strip()))
    return found


def test_parser_flags_a_register_amount():
    text = ("0000000000001000 <k>:\n"
            "\tv_lshlrev_b64 v[12:13], v15, s[0:1]   // 0001\n"
            "\tv_lshlrev_b64 v[2:3], 1, v[0:1]        // 0002\n"
            "\tv_lshrrev_b64 v[4:5], s2, v[4:5]       // 0003\n")
    assert shift64_by_register(text) == [("k", "v_lshlrev_b64 v[12:13], v15, s[0:1]")]


def test_no_64bit_shift_by_a_register_amount(tmp_path):
    dis = _disassemble(tmp_path)
    assert "v_" in dis
    bad = shift64_by_register(dis)
    assert not bad, "64-bit shifts by a VGPR amount:\n" + "\n".join(f"{f}: {i}" for f, i in bad[:20])
