"""Host-side checks of bench.py: the algorithmic byte counts it divides by and
its refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_layer_bytes_match_the_counted_rows():
    # full layer at 64 x 4096, bf16: K and V rows of 64 streams x 8 kv heads x
    # 4096 keys x 256 dims x 2 bytes, plus per stream q in and out (2 x 8 x
    # 256 x 4), k and v in (2 x 8 x 256 x 4), the rounded entry out (2 x 8 x
    # 256 x 2), gate logits (8 x 4) and pos (4)
    per_stream = 2 * 8 * 256 * 4 + 2 * 8 * 256 * 4 + 2 * 8 * 256 * 2 + 8 * 4 + 4
    assert bench.layer_bytes("full") == 64 * 8 * 4096 * 256 * 2 * 2 + 64 * per_stream
    assert bench.layer_bytes("sliding") == 64 * 8 * 511 * 256 * 2 * 2 + 64 * per_stream
    assert round(bench.layer_bytes("full") / 1e6, 1) == 2150.1
    assert round(bench.layer_bytes("sliding") / 1e6, 1) == 270.5
    step = 21 * bench.layer_bytes("sliding") + 7 * bench.layer_bytes("full")
    assert round(step / 1e9, 2) == 20.73
    # fp8: one byte per cached element, plus the 2 x 8 per-head scales
    assert bench.layer_bytes("full", elt=1) == (64 * 8 * 4096 * 256 * 2
                                                + 64 * (per_stream - 2 * 8 * 256) + 2 * 8 * 4)
    # grouped: 32 query heads over the same 8 kv heads add only query-side I/O
    assert (bench.layer_bytes("full", heads=32) - bench.layer_bytes("full")
            == 64 * (24 * 256 * 4 * 2 + 24 * 4))


def test_interleave_has_seven_full_layers():
    full = [l for l in range(bench.LAYERS) if bench.is_full(l)]
    assert full == [3, 7, 11, 15, 19, 23, 27]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_traffic_is_close_to_the_algorithmic_bytes():
    """Where the committed counters match the kernel code, the measured HBM
    bytes of the full-layer launch are within a few percent of what the
    method must move (more would mean re-reads; less, a miscount).  A group
    split into pieces reads the cache once per piece at most."""
    for kv, elt in (("bf16", 2), ("fp8", 1)):
        for heads in (8, 16, 24, 32, 64):
            t = bench.measured_traffic(kv, heads)
            if t is None:
                continue
            alg = bench.layer_bytes("full", elt=elt, heads=heads)
            pieces = bench.kernel_group(kv, heads)[1]
            assert 0.999 * alg <= t <= 1.03 * pieces * alg, (kv, heads, t, alg)


def test_kernel_group():
    assert bench.kernel_group("bf16", 8) == (1, 1)
    assert bench.kernel_group("bf16", 16) == (2, 1)
    assert bench.kernel_group("bf16", 24) == (4, 1)
    assert bench.kernel_group("bf16", 64) == (4, 2)
    assert bench.kernel_group("fp8", 64) == (8, 1)
    assert bench.full_kernel("bf16", 64) == "hswd::attn_kernel<256, 2, false, 1, 4, true>(...)"
    assert bench.full_kernel("fp8", 8) == "hswd::attn_kernel<256, 3, false, 1, 1, false>(...)"
