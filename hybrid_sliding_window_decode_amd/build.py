"""Build libhswd.so (HIP, gfx950) in-tree.

    python -m hybrid_sliding_window_decode_amd.build

Translation units: csrc/hswd.hip (host entry points and the small kernels)
and csrc/attn_g{1,2,4,8}.hip (the attention kernel for 1, 2, 4 or 8 query heads
per kv head; attn_g8s.hip: its form for the pieces of larger groups),
compiled in parallel with hipcc for gfx950 only and linked into one shared
library; csrc/measure.hip (the streaming-read probe the benchmark compares
the kernels with) into libhswd_measure.so beside it.  Packed fp32 instructions are turned off
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
MEASURE_SRC = os.path.join(CSRC, "measure.hip")
MEASURE_LIB = os.path.join(HERE, "libhswd_measure.so")
DEPS = (SOURCES + [MEASURE_SRC] + sorted(glob.glob(os.path.join(CSRC, "*.hpp")))
        + sorted(glob.glob(os.path.join(CSRC, "kernels", "*.hpp")))
        + [os.path.join(ROOT, "include", "hswd.h"), os.path.join(ROOT, "include", "hswd_measure.h")])

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def build(out=LIB, extra=(), verbose=False, jobs=7):
    """Compile and link libhswd.so at `out` and libhswd_measure.so beside it."""
    measure_out = os.path.join(os.path.dirname(os.path.abspath(out)), os.path.basename(MEASURE_LIB))
    srcs = SOURCES + [MEASURE_SRC]
    with tempfile.TemporaryDirectory(prefix="hswd_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]

        def run(cmd):
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            subprocess.run(cmd, check=True)

        def compile_one(pair):
            src, obj = pair
            run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(compile_one, zip(srcs, objs)))
        tmps = []
        for target, parts in ((out, objs[:-1]), (measure_out, objs[-1:])):
            tmp = target + ".tmp%d" % os.getpid()
            run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *parts, "-o", tmp])
            tmps.append((tmp, target))
    for tmp, target in tmps:
        os.replace(tmp, target)
    return out


def stale():
    if not (os.path.exists(LIB) and os.path.exists(MEASURE_LIB)):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(MEASURE_LIB))
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(extra=extra, verbose=True))
