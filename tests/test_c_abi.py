"""The C ABI from C: include/nm_mask.h compiles as strict C99 with warnings as errors and no HIP
or C++ headers, and a C program linked against libnm_mask.so gets the host helpers' answers and
the host-side argument validation (no GPU needed: nothing it calls reaches the device)."""
import os
import shutil
import subprocess

import pytest

import semi_structured_sparsity_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_host_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c99_and_host_calls_work(tmp_path):
    lib = S.library_path()
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_host_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic-errors", "-Wno-error=pedantic",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", str(exe),
           "-L", os.path.dirname(lib), "-l:" + os.path.basename(lib), "-Wl,-rpath," + os.path.dirname(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi host check: ok" in run.stdout
