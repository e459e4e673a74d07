"""Build tests/c_abi/layer_step, the C-ABI caller the GPU test
tests/test_gpu_c_abi.py runs: host code only (hipcc for the HIP runtime
headers), linked against the in-tree libhswd.so (found through its rpath)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "layer_step.cpp")
EXE = os.path.join(HERE, "layer_step")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build():
    libdir = os.path.join(ROOT, "hybrid_sliding_window_decode_amd")
    tmp = EXE + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "-O2", "-std=c++17", SRC, "-o", tmp, "-L" + libdir, "-lhswd",
                    "-Wl,-rpath,$ORIGIN/../../hybrid_sliding_window_decode_amd"], check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
