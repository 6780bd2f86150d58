"""Build libnm_mask.so, the HIP library behind include/nm_mask.h, for gfx950 (MI355X).

hipcc cross-compiles the device code, so the library builds on a host without a GPU.  Packed
FP32 instructions are disabled for all device code (-packed-fp32-ops).
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("nm_forward.hip", "nm_backward.hip", "nm_backward_wreg.hip", "nm_pack.hip", "nm_spmm.hip",
            "nm_abi.hip")]
HEADERS = [os.path.join(CSRC, "nm_device.hpp"), os.path.join(CSRC, "nm_layer.hpp"),
           os.path.join(CSRC, "nm_backward.hpp"),
           os.path.join(CSRC, "nm_kernels.hpp"), os.path.join(ROOT, "include", "nm_mask.h")]
LIB = os.path.join(PKG, "libnm_mask.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
# -Wall is left out of the default flags: it doubles the device compile time of the fully
# unrolled kernels (4.5 instead of 2 minutes for the backward's translation unit).
# Per-source flags: the monitored forward's tree atomics are issued by one lane, so the
# compiler's wave-level atomic combining (which would wait for each of a block's two adds
# alone) is turned off for that file.
SOURCE_FLAGS = {"nm_forward.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(noise))
    return noise


def build(out=LIB, verbose=False):
    """Compile the library (always, even if it exists) and return its path.  Each translation
    unit is compiled on its own hipcc process, in parallel, then the objects are linked."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, ["hipcc", *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", "-o", o, src])
                for src, o in zip(SOURCES, objs)]
        noise = [l for f in futs for l in f.result()]
    tmp = out + ".tmp"
    noise += _run(["hipcc", *FLAGS, "-shared", "-o", tmp, *objs])
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
