"""hswd_layer_step_noalloc (the entry point that allocates nothing, its
workspace in the library's own per-GPU array) against hswd_layer_step with a
workspace of its own: the same kernels and the same chunking, so the same
bits.  Calls come in a row, each later one smaller than the one before, so
what an earlier call left in the shared array (partials, counters) is there
when the next one runs; cross-workgroup merges, a group split into head
pieces and the error flags are covered."""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def _compare(spec, pos, seed, max_pos=None):
    x = inputs.make_step(spec, pos, seed)
    a, b = to_dev(x), to_dev(x)                 # identical inputs and caches
    ring = spec.kind == "sliding"
    mp = int(np.max(x.pos)) if max_pos is None else max_pos
    desc = hswd.make_desc(a["k_cache"], n_heads=spec.H, kv_scale=a["kv_scale"])
    ws = hswd.workspace(desc, ring, mp)
    n_split = hswd.num_splits(desc, ring, mp)
    say("noalloc vs layer_step: %s %s B=%d H=%d Hkv=%d pos=%s, %d chunks, workspace %d B" % (
        spec.kind, spec.dtype, spec.B, spec.H, spec.Hkv, list(x.pos[:4]), n_split, ws.numel()))
    want = hswd.layer_step(a["q"], a["k"], a["v"], a["gate"], a["k_cache"], a["v_cache"],
                           a["pos"], ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full_like(b["q"], float("nan"))
    got = hswd.layer_step_noalloc(b["q"], b["k"], b["v"], b["gate"], b["k_cache"], b["v_cache"],
                                  b["pos"], ring, spec.rot, spec.theta, max_pos=mp, out=out,
                                  desc=desc, err=err)
    assert got is out
    flags_ws = hswd.check_errors(ws)
    flags = hswd.check_errors(err)
    assert flags == flags_ws, (flags, flags_ws)
    assert torch.equal(_bits(got), _bits(want)), float((got - want).abs().max())
    assert torch.equal(_bits(b["k_cache"]), _bits(a["k_cache"]))
    assert torch.equal(_bits(b["v_cache"]), _bits(a["v_cache"]))
    return flags


def test_noalloc_equals_layer_step_on_calls_in_a_row():
    # 1: 4 streams near 20000 keys: several workgroups per (stream, kv head),
    #    chunk partials and arrival counters in the array
    big = inputs.full_spec(4, 20001, "bf16")
    assert _compare(big, [20000, 19000, 7777, 20000], 71) == 0
    # 2: smaller, 2 streams near 9000: other chunks, other partial offsets
    assert _compare(inputs.full_spec(2, 9001, "bf16"), [9000, 8191], 72) == 0
    # 3: smaller again, 128 query heads over 8 kv heads in two pieces of
    #    eight per group (entry-write arrival counters)
    assert _compare(inputs.full_spec(1, 4097, "bf16", H=128), [4096], 73) == 0
    # 4: a ring, f32, one stream
    assert _compare(inputs.sliding_spec(1, "f32"), [600], 74) == 0
    # 5: error flags through the caller's word: a stream past the grid's
    #    max_pos and at the capacity (write skipped)
    f = _compare(inputs.full_spec(2, 3001, "f16"), [3001, 100], 75, max_pos=3000)
    assert f == (hswd.binding.FLAG_CAPACITY | hswd.binding.FLAG_MAX_POS), f
    # 6: the first call again: the array holds what the calls above left
    assert _compare(big, [20000, 19000, 7777, 20000], 76) == 0


def test_noalloc_fp8_grouped():
    """An fp8 cache with per-head scales and 32 query heads (the 4-head
    matrix-core kernel) over several workgroups per kv head."""
    assert _compare(inputs.full_spec(2, 12001, "fp8", H=32), [12000, 11000], 77) == 0
    assert _compare(inputs.sliding_spec(3, "fp8", H=32), [4096, 100, 511], 78) == 0
