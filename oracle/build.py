"""Compile the CPU oracle (plain C, gcc) into oracle/libnm_oracle.so.

Test infrastructure: the oracle is the checker of the HIP library, not part of it.  The flags
keep IEEE binary64 semantics exactly as written in the source: no fast-math and no contraction
of a*b+c into a fused multiply-add.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nm_oracle.c")
LIB = os.path.join(HERE, "libnm_oracle.so")
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(out=LIB, src=SRC, extra=(), quiet=False):
    """Compile `src` to the shared library `out`; returns the path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if res.stderr and not quiet:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
