"""The constants the pages fix, as stored in tests/golden/page_constants.json
(each with its citation), against every place they reach the computation:
the layer specs of inputs.py (which the oracle's pins, the GPU tests and the
benchmark all build their layers from), the 3:1 interleave, bench.py's
workload constants and the gate projection's shape.  A wrong value in one of
them would otherwise flow identically into the oracle, the GPU path and the
benchmark, and no parity check could see it.  CPU only."""
import json
import os
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hybrid_sliding_window_decode_amd import inputs  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "page_constants.json")


def load():
    return json.load(open(GOLDEN))


def check_constants(c, inp, bn):
    """Raise AssertionError where `inp` (the inputs module) or `bn` (the bench
    module) disagrees with the page constants `c`."""
    D, H = c["heads"]["head_dim"], c["heads"]["n_heads"]
    S = c["ring_slots"]["value"]
    # the window counts the current token: the ring keeps window - 1 entries
    assert S == c["window"]["value"] - 1
    for dt in ("f32", "f16", "bf16", "fp8"):
        s = inp.sliding_spec(4, dt)
        assert (s.kind, s.n_slots, s.H, s.D) == ("sliding", S, H, D), (dt, s)
        assert (s.rot, s.theta) == (c["sliding_rope"]["rot_dim"], c["sliding_rope"]["theta"]), s
        f = inp.full_spec(4, 4097, dt)
        assert (f.kind, f.n_slots, f.H, f.D) == ("full", 4097, H, D), (dt, f)
        assert (f.rot, f.theta) == (c["full_rope"]["rot_dim"], c["full_rope"]["theta"]), f
    # full layers rotate the first quarter of the head dims
    assert c["full_rope"]["rot_dim"] * 4 == D
    assert c["sliding_rope"]["rot_dim"] == D
    # 3 sliding per full layer, 21 + 7 over 28 layers, in inputs and in bench
    il = c["interleave"]
    n = il["layers"]
    full = [l for l in range(n) if inp.layer_is_full(l)]
    assert len(full) == il["full_layers"] and n - len(full) == il["sliding_layers"]
    for p in range(0, n, il["sliding_per_full"] + 1):
        period = [inp.layer_is_full(l) for l in range(p, p + il["sliding_per_full"] + 1)]
        assert sum(period) == 1, (p, period)
    assert bn.LAYERS == n
    assert [bn.is_full(l) for l in range(n)] == [inp.layer_is_full(l) for l in range(n)]
    assert (bn.S_RING, bn.H, bn.HKV, bn.D) == (S, H, H, D)
    # the gate [hidden, heads] = [2048, 8]; its weight is stored a row per head
    hidden, heads = c["gate_weight_shape"]["value"]
    assert heads == H
    x, w = inp.gate_inputs(3, hidden, heads, seed=1)
    assert x.shape == (3, hidden) and w.shape == (heads, hidden)


def test_page_constants_reach_every_layer_spec():
    check_constants(load(), inputs, bench)


def test_bench_step_uses_the_page_specs():
    """The benchmark's 28-layer step builds each layer from these specs."""
    c = load()
    for l in range(bench.LAYERS):
        spec = (inputs.full_spec(bench.B, bench.CTX + 1, "bf16") if bench.is_full(l)
                else inputs.sliding_spec(bench.B, "bf16"))
        want = c["full_rope"] if bench.is_full(l) else c["sliding_rope"]
        assert (spec.rot, spec.theta) == (want["rot_dim"], want["theta"])


def _patched(name, fn):
    """A stand-in for the inputs module with one function replaced."""
    ns = SimpleNamespace(**{k: getattr(inputs, k) for k in dir(inputs) if not k.startswith("__")})
    setattr(ns, name, fn)
    return ns


def _wrap(orig, **changes):
    def f(*a, **kw):
        s = orig(*a, **kw)
        for k, v in changes.items():
            setattr(s, k, v)
        return s
    return f


MUTANTS = [
    ("sliding theta 1e5", "sliding_spec", _wrap(inputs.sliding_spec, theta=1e5)),
    ("full theta 1e4", "full_spec", _wrap(inputs.full_spec, theta=1e4)),
    ("ring of 512 slots", "sliding_spec", _wrap(inputs.sliding_spec, n_slots=512)),
    ("full layers rotate half the dims", "full_spec", _wrap(inputs.full_spec, rot=128)),
    ("sliding layers rotate a quarter", "sliding_spec", _wrap(inputs.sliding_spec, rot=64)),
    ("1:1 interleave", "layer_is_full", lambda l: l % 2 == 1),
    ("gate weight [hidden, heads] layout", "gate_inputs",
     lambda B, hidden, H, seed: (inputs.gate_inputs(B, hidden, H, seed)[0],
                                 inputs.gate_inputs(B, hidden, H, seed)[1].T)),
]


@pytest.mark.parametrize("name,fn_name,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_constant_mutant_is_rejected(name, fn_name, fn):
    with pytest.raises(AssertionError):
        check_constants(load(), _patched(fn_name, fn), bench)


def test_bench_mutant_is_rejected():
    bn = SimpleNamespace(**{k: getattr(bench, k) for k in ("LAYERS", "S_RING", "H", "HKV", "D")})
    bn.is_full = lambda l: l % 4 == 0          # same count, different layers than inputs
    with pytest.raises(AssertionError):
        check_constants(load(), inputs, bn)
