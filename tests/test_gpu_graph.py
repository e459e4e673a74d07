"""A captured HIP graph of layer steps replays to the eager results.

The layer step launches kernels only (no memset, no allocation; the
cross-workgroup arrival counters reset themselves), so a whole decode step
can be captured once and replayed.  Each replay is checked against the
eager outputs and cache contents, with eager work and synchronisations
between replays.  Positions are chosen so that a step's own entry write
does not change what the next replay attends (rings not yet wrapped, append
rows past the valid range), which makes every replay equal to the first."""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import cache_to_host, say

pytestmark = pytest.mark.gpu


def make_layers(seed):
    layers = []
    for i, (kind, dtype, H) in enumerate([("sliding", "bf16", 8), ("full", "bf16", 8),
                                          ("full", "fp8", 8), ("sliding", "bf16", 32),
                                          ("full", "f16", 16), ("full", "fp8", 32),
                                          ("sliding", "fp8", 64), ("full", "bf16", 64)]):
        B = 6
        if kind == "sliding":
            spec = inputs.sliding_spec(B, dtype, H=H)
            pos = inputs.ragged_positions(B, 1, 510, seed=seed + i)
        else:
            spec = inputs.full_spec(B, 3000, dtype, H=H)
            pos = inputs.ragged_positions(B, 1, 2999, seed=seed + i)
        # six streams leave room for several workgroups per kv head on the
        # append caches (the cross-workgroup merge)
        t = inputs.device_step(spec, pos, seed=seed + 10 + i)
        t["desc"] = hswd.make_desc(t["k_cache"], n_heads=H, kv_scale=t.get("kv_scale"))
        t["spec"] = spec
        t["ring"] = kind == "sliding"
        t["mp"] = int(t["pos"].max())
        t["ws"] = hswd.workspace(t["desc"], t["ring"], t["mp"])
        t["out"] = torch.empty_like(t["q"])
        layers.append(t)
    return layers


def step(layers):
    for t in layers:
        hswd.layer_step(t["q"], t["k"], t["v"], t["gate"], t["k_cache"], t["v_cache"], t["pos"],
                        t["ring"], t["spec"].rot, t["spec"].theta, t["ws"], max_pos=t["mp"],
                        out=t["out"], desc=t["desc"])


def test_graph_replays_equal_eager():
    layers = make_layers(70)
    say("graph: eager reference")
    step(layers)
    torch.cuda.synchronize()
    ref_out = [t["out"].clone() for t in layers]
    ref_k = [cache_to_host(t["k_cache"]) for t in layers]
    for t in layers:
        assert hswd.check_errors(t["ws"]) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(layers)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(layers)
    other = make_layers(90)                      # eager work between replays
    for r in range(4):
        for t in layers:
            t["out"].fill_(float("nan"))
        say("graph: replay %d" % r)
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(layers):
            assert torch.equal(t["out"], ref_out[i]), (r, i)
            assert np.array_equal(cache_to_host(t["k_cache"]), ref_k[i]), (r, i)
        step(other)
        torch.cuda.synchronize()
    for t in layers + other:
        assert hswd.check_errors(t["ws"]) == 0
