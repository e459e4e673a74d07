"""AddressSanitizer and UndefinedBehaviorSanitizer builds on the CPU.

* The oracle: tests/sanitize/oracle_driver.c compiles the oracle's C source
  with gcc's sanitizers (leak checking on) and calls every public function
  on small cases that reach its edges.
* The host side of libhswd: hswd.hip (argument checks, chunking, workspace
  layout, dispatch) and the measurement library's measure.hip, built with
  the sanitizers on their host code only, linked
  with stub attention launchers (tests/sanitize/attn_launch_stub.hip) so the
  attention kernels need not be compiled, and driven through every entry
  point's host checks by tests/sanitize/abi_driver.c.  Without a GPU, valid
  calls come back as HSWD_ERR_HIP; leak checking is off for this one, since
  the HIP runtime keeps its own allocations until exit.

A sanitizer report makes the driver exit non-zero, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
CSRC = os.path.join(ROOT, "hybrid_sliding_window_decode_amd", "csrc")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
# sanitizers on host code only: each -fsanitize flag right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=gnu11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=300)
    assert "oracle sanitizer driver: ok" in r.stdout


def test_library_host_side_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    t = str(tmp_path)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN
    objs = []
    for src, obj in [(os.path.join(CSRC, "hswd.hip"), "hswd.o"),
                     (os.path.join(CSRC, "measure.hip"), "measure.o"),
                     (os.path.join(SAN, "attn_launch_stub.hip"), "stub.o")]:
        _run([HIPCC] + flags + ["-c", src, "-o", os.path.join(t, obj)])
        objs.append(os.path.join(t, obj))
    drv = os.path.join(t, "abi_driver.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = os.path.join(t, "abi_san")
    _run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN[:4] + [drv] + objs + ["-o", exe])
    # no device is ever visible to this driver, even on a host with a GPU:
    # its pointers are stand-ins
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = _run([exe], env=env, timeout=120)
    assert "abi sanitizer driver: ok" in r.stdout
