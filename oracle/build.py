"""Builds the oracle's shared library (test infrastructure only).

`python -m oracle.build` compiles `oracle/hswd_oracle.c` with gcc into
`oracle/liboracle.so`.  Plain C, fp64, OpenMP over (stream, head); no HIP.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hswd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
