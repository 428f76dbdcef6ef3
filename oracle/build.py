"""Compile the CPU oracle (test infrastructure) into oracle/libgdn_oracle.so.

Plain gcc, double precision, no fast-math and no FMA contraction, so the
oracle's rounding follows the order written in gdn_oracle.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
          "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
