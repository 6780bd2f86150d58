"""The host code under the compilers' sanitizers, on the CPU (no GPU is used or needed):

* the oracle (oracle/nm_oracle.c) driven by tests/c/oracle_sanitize.c, built with gcc's
  AddressSanitizer + UndefinedBehaviorSanitizer, then with ThreadSanitizer (the oracle splits
  rows over pthreads; the driver runs 1, 3 and 8 workers);
* the library's host code (the C ABI's argument checks and size arithmetic in nm_abi.hip and the
  launchers' host side in every .hip source) built with ASan + UBSan on the host side only, and
  driven by tests/c/abi_host_check.c, whose every call is answered on the host before any HIP
  call (extreme shapes, token counts and samples among them).

Any sanitizer report fails the test (the runtimes are told to stop at the first one).  GPU code
is never built with a sanitizer: the device side of the library keeps its own flags, at -O1
here because it is only linked, never run."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "nm_oracle.c")
ORACLE_DRIVER = os.path.join(ROOT, "tests", "c", "oracle_sanitize.c")
ABI_DRIVER = os.path.join(ROOT, "tests", "c", "abi_host_check.c")
CSRC = os.path.join(ROOT, "semi_structured_sparsity_amd", "csrc")
HIP_SOURCES = ["nm_forward.hip", "nm_backward.hip", "nm_backward_wreg.hip", "nm_pack.hip", "nm_spmm.hip",
               "nm_abi.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

ORACLE_FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", "-ffp-contract=off",
                "-fno-fast-math", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "oracle")]
# Host side only: each sanitizer flag goes to the host compilation.
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
HOST_NO_RECOVER = "-Xarch_host -fno-sanitize-recover=all".split()
HIP_FLAGS = ["-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-O1", "-Xarch_device", "-O1",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-omit-frame-pointer",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
ASAN_ENV = {"ASAN_OPTIONS": "verify_asan_link_order=0:halt_on_error=1:detect_leaks=1",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-3000:] + res.stderr[-3000:]
    return res


def _execute(exe, env_extra, marker):
    env = dict(os.environ, **env_extra)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert marker in res.stdout, report
    for word in ("runtime error", "Sanitizer", "WARNING: ThreadSanitizer"):
        assert word not in res.stderr, report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("kind", ["address,undefined", "thread"])
def test_oracle_under_sanitizers(tmp_path, kind):
    exe = tmp_path / "oracle_sanitize"
    extra = ["-fno-sanitize-recover=all"] if "undefined" in kind else []
    _run(["gcc", *ORACLE_FLAGS, f"-fsanitize={kind}", *extra, ORACLE_SRC, ORACLE_DRIVER, "-lm", "-o", str(exe)])
    env = ASAN_ENV if kind != "thread" else {"TSAN_OPTIONS": "halt_on_error=1"}
    _execute(exe, env, "oracle sanitize check: ok")


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANGXX), reason="needs hipcc and ROCm clang")
def test_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    objs = [tmp_path / (src + ".o") for src in HIP_SOURCES]
    jobs = min(len(HIP_SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, ["hipcc", *HIP_FLAGS, *HOST_SANITIZE, *HOST_NO_RECOVER, "-c",
                                 os.path.join(CSRC, src), "-o", str(o)]) for src, o in zip(HIP_SOURCES, objs)]
        for f in futs:
            f.result()
    check = tmp_path / "abi_host_check.o"
    _run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", ABI_DRIVER, "-o", str(check)])
    exe = tmp_path / "abi_sanitize"
    _run([CLANGXX, "-fsanitize=address,undefined", str(check), *map(str, objs), "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)])
    # the HIP runtime's own allocations at exit are not this library's: leaks are not checked here
    env = dict(ASAN_ENV, ASAN_OPTIONS="verify_asan_link_order=0:halt_on_error=1:detect_leaks=0")
    _execute(exe, env, "abi host check: ok")
