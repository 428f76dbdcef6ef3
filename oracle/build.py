"""Compile the CPU oracles (test infrastructure): oracle/libgdn_oracle.so (the
recurrence) and oracle/libgdn_preprocess.so (the pre-processing in front of it).

Plain gcc, double precision, no fast-math and no FMA contraction, so the
oracle's rounding follows the order written in gdn_oracle.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")
PRE_SRC = os.path.join(HERE, "gdn_preprocess.c")
PRE_LIB = os.path.join(HERE, "libgdn_preprocess.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
          "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`.  With the
    default arguments the pre-processing oracle is built as well."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if src == SRC and out == LIB and not extra:
        build(PRE_SRC, PRE_LIB)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
