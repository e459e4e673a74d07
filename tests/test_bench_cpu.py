"""Host-side checks of bench.py: the algorithmic byte counts it divides by and
its refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

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


HEADLINE_COUNTERS = [("bf16", 8), ("fp8", 8)]
OTHER_COUNTERS = [(kv, h) for kv in ("bf16", "fp8") for h in (16, 24, 32, 64)]


def _check_traffic(kv, heads):
    elt = 1 if kv == "fp8" else 2
    t = bench.measured_traffic(kv, heads)
    alg = bench.layer_bytes("full", elt=elt, heads=heads)
    pieces = bench.kernel_group(kv, heads)[1]
    assert 0.999 * alg <= t <= 1.03 * pieces * alg, (kv, heads, t, alg)


@pytest.mark.parametrize("kv,heads", HEADLINE_COUNTERS)
def test_headline_counters_match_the_kernel_code(kv, heads):
    """The committed FETCH_SIZE / WRITE_SIZE counters of the benchmark's own
    steps (8 query heads, bf16 and fp8 caches) must have been taken on the
    current device code: bench.py reports roofline.traffic from them, so a
    kernel change must come with new counters."""
    assert os.path.exists(bench.counters_path(kv, heads)), "no committed counters"
    assert bench.measured_traffic(kv, heads) is not None, (
        "profiles/%s is older than the kernel code: re-take FETCH_SIZE and "
        "WRITE_SIZE" % os.path.basename(bench.counters_path(kv, heads)))
    # the measured HBM bytes of the full-layer launch are within a few
    # percent of what the method must move (more would mean re-reads; less,
    # a miscount)
    _check_traffic(kv, heads)


@pytest.mark.parametrize("kv,heads", OTHER_COUNTERS)
def test_grouped_counters_close_to_the_algorithmic_bytes(kv, heads):
    """Grouped steps: where committed counters match the kernel code, their
    traffic is within a few percent of the algorithmic bytes (a group split
    into pieces reads the cache once per piece at most)."""
    if not os.path.exists(bench.counters_path(kv, heads)):
        pytest.skip("no committed counters for %s with %d query heads" % (kv, heads))
    if bench.measured_traffic(kv, heads) is None:
        pytest.skip("committed counters for %s with %d query heads predate the kernel "
                    "code" % (kv, heads))
    _check_traffic(kv, heads)


def test_kernel_group():
    assert bench.kernel_group("bf16", 8) == (1, 1)
    assert bench.kernel_group("bf16", 16) == (2, 1)
    assert bench.kernel_group("bf16", 24) == (4, 1)
    assert bench.kernel_group("bf16", 64) == (8, 1)
    assert bench.kernel_group("bf16", 40) == (8, 1)
    assert bench.kernel_group("fp8", 64) == (8, 1)
    assert bench.kernel_group("fp8", 16) == (4, 1)
    assert bench.kernel_group("bf16", 16) == (2, 1)
    assert bench.full_kernel("bf16", 64) == "hswd::attn_kernel<256, 2, false, 1, 8, false>(...)"
    assert bench.full_kernel("fp8", 8) == "hswd::attn_kernel<256, 3, false, 1, 1, false>(...)"
