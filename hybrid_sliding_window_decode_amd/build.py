"""Build libhswd.so (HIP, gfx950) in-tree.

    python -m hybrid_sliding_window_decode_amd.build

Translation units: csrc/hswd.hip (host entry points and the small kernels)
and csrc/attn_g{1,2,4,8}.hip (the attention kernel for 1, 2, 4 or 8 query heads
per kv head; attn_g8s.hip: its form for the pieces of larger groups),
compiled in parallel with hipcc for gfx950 only and linked into one shared
library.  Packed fp32 instructions are turned off
(-packed-fp32-ops): the kernels are written for scalar fp32 VALU ops.
"""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("hswd.hip", "attn_g1.hip", "attn_g2.hip",
                                            "attn_g4.hip", "attn_g8.hip", "attn_g8s.hip")]
SRC = SOURCES[0]
LIB = os.path.join(HERE, "libhswd.so")
DEPS = (SOURCES + sorted(glob.glob(os.path.join(CSRC, "*.hpp")))
        + sorted(glob.glob(os.path.join(CSRC, "kernels", "*.hpp")))
        + [os.path.join(ROOT, "include", "hswd.h")])

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def build(out=LIB, extra=(), verbose=False, jobs=7):
    with tempfile.TemporaryDirectory(prefix="hswd_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]

        def compile_one(pair):
            src, obj = pair
            cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(compile_one, zip(SOURCES, objs)))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
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
