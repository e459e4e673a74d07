"""Build libhswd.so (HIP, gfx950) in-tree.

    python -m hybrid_sliding_window_decode_amd.build

One translation unit, csrc/hswd.hip, compiled with hipcc for gfx950 only.
Packed fp32 instructions are turned off (-packed-fp32-ops): the kernels are
written for scalar fp32 VALU ops.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "hswd.hip")
LIB = os.path.join(HERE, "libhswd.so")
DEPS = [SRC, os.path.join(HERE, "csrc", "kernels", "attn.hpp"),
        os.path.join(HERE, "csrc", "kernels", "common.hpp"),
        os.path.join(HERE, "csrc", "kernels", "small.hpp"),
        os.path.join(ROOT, "include", "hswd.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def build(out=LIB, extra=(), verbose=False):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(extra=extra, verbose=True))
