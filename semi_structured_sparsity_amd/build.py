"""Build libnm_mask.so, the HIP library behind include/nm_mask.h, for gfx950 (MI355X).

hipcc cross-compiles the device code, so the library builds on a host without a GPU.  Packed
FP32 instructions are disabled for all device code (-packed-fp32-ops).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "nm_kernels.hip"), os.path.join(CSRC, "nm_spmm.hip"),
           os.path.join(CSRC, "nm_abi.hip")]
HEADERS = [os.path.join(CSRC, "nm_device.hpp"), os.path.join(CSRC, "nm_kernels.hpp"),
           os.path.join(ROOT, "include", "nm_mask.h")]
LIB = os.path.join(PKG, "libnm_mask.so")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def build(out=LIB, verbose=False):
    """Compile the library (always, even if it exists) and return its path."""
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(noise))
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, out)
    return out


def stale(out=LIB):
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
