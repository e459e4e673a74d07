"""Safety nets on the GPU.

* Guard canaries: every buffer a fused layer step writes or reads (the
  output, the workspace, both caches, and the q/k/v/gate inputs) sits inside
  a larger allocation whose margins hold a fixed byte pattern; after the
  step the margins must be intact and the inputs unchanged.  Cases cover one
  workgroup per (stream, kv head), the cross-workgroup merge (partials and
  arrival counters in the workspace), a group split into head pieces, and
  the entry point with the library's own workspace.
* Checkpoint and resume: a run of decode steps through the ring's wrap is
  interrupted, its caches copied to the host and restored into fresh device
  buffers with a fresh workspace, and continued; every later output and the
  final caches must equal the uninterrupted run's bit for bit.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import TORCH_DT, say

pytestmark = pytest.mark.gpu

PAD = 1 << 16             # bytes of margin on each side of a guarded buffer
PATTERN = 0xA5


def _bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


class Guarded:
    """A tensor of `shape` / `dtype` in the middle of a byte allocation whose
    PAD-byte margins hold PATTERN."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((PAD + n + PAD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[PAD:PAD + n].view(dtype).view(*shape)
        if fill is not None:
            _bits(self.t).copy_(_bits(fill.to("cuda").view(dtype)))

    def margins_intact(self):
        return bool((self.raw[:PAD] == PATTERN).all() and (self.raw[-PAD:] == PATTERN).all())


def _guarded_step(spec, pos, seed, noalloc=False):
    x = inputs.make_step(spec, pos, seed)
    dt = TORCH_DT[spec.dtype]
    ring = spec.kind == "sliding"
    B, H, Hkv, D, S = spec.B, spec.H, spec.Hkv, spec.D, spec.n_slots
    host = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    cache_host = lambda a: host(a.view(np.int16) if a.dtype == np.uint16 else a)
    q = Guarded((B, H, D), torch.float32, host(x.q))
    k = Guarded((B, Hkv, D), torch.float32, host(x.k))
    v = Guarded((B, Hkv, D), torch.float32, host(x.v))
    g = Guarded((B, H), torch.float32, host(x.gate))
    kc = Guarded((B, Hkv, S, D), dt, cache_host(x.k_cache))
    vc = Guarded((B, Hkv, S, D), dt, cache_host(x.v_cache))
    out = Guarded((B, H, D), torch.float32)
    pos_t = torch.from_numpy(x.pos).cuda()
    kv_scale = None if spec.kv_scale is None else torch.from_numpy(spec.kv_scale).cuda()
    desc = hswd.make_desc(kc.t, n_heads=H, kv_scale=kv_scale)
    mp = int(np.max(x.pos))
    n_ws = hswd.workspace_bytes(desc, ring, mp)
    ws = Guarded((n_ws,), torch.uint8)
    hswd.workspace_init(ws.t)
    before = {n: _bits(b.t).clone() for n, b in (("q", q), ("k", k), ("v", v), ("gate", g))}
    say("canaries: %s %s B=%d H=%d Hkv=%d pos=%s %s, %d chunks" % (
        spec.kind, spec.dtype, B, H, Hkv, list(x.pos), "noalloc" if noalloc else "workspace",
        hswd.num_splits(desc, ring, mp)))
    if noalloc:
        hswd.layer_step_noalloc(q.t, k.t, v.t, g.t, kc.t, vc.t, pos_t, ring, spec.rot,
                                spec.theta, max_pos=mp, out=out.t, desc=desc)
    else:
        hswd.layer_step(q.t, k.t, v.t, g.t, kc.t, vc.t, pos_t, ring, spec.rot, spec.theta, ws.t,
                        max_pos=mp, out=out.t, desc=desc)
        assert hswd.check_errors(ws.t) == 0
    torch.cuda.synchronize()
    for name, b in (("q", q), ("k", k), ("v", v), ("gate", g), ("k_cache", kc),
                    ("v_cache", vc), ("out", out), ("workspace", ws)):
        assert b.margins_intact(), "a write landed outside %s" % name
    for n, b in (("q", q), ("k", k), ("v", v), ("gate", g)):
        assert torch.equal(_bits(b.t), before[n]), "%s was modified" % n
    assert torch.isfinite(out.t).all()


@pytest.mark.parametrize("noalloc", [False, True])
def test_canaries_around_every_buffer(noalloc):
    # one workgroup per (stream, kv head): 64 rings
    _guarded_step(inputs.sliding_spec(64, "bf16"), inputs.ragged_positions(64, 1, 4096, 3), 81,
                  noalloc)
    # cross-workgroup merges: few streams, long append caches
    _guarded_step(inputs.full_spec(3, 9001, "f16"), [9000, 4097, 1], 82, noalloc)
    # a group split into head pieces (entry arrival counters)
    _guarded_step(inputs.full_spec(2, 4097, "bf16", H=128), [4096, 3000], 83, noalloc)
    # the 8-head kernel over a 16-bit cache (partials flushed in two halves)
    _guarded_step(inputs.full_spec(2, 9001, "bf16", H=64), [9000, 4097], 86, noalloc)
    # fp8 with per-head scales, 4-head matrix-core kernel, ring
    _guarded_step(inputs.sliding_spec(2, "fp8", H=32), [600, 7], 84, noalloc)
    # f32 ring, one stream
    _guarded_step(inputs.sliding_spec(1, "f32"), [600], 85, noalloc)


def _run_steps(layers, steps, first, last, state):
    """Steps first..last-1 of every layer from `state` (device caches and
    workspaces per layer); returns the outputs per (step, layer)."""
    outs = {}
    for s in range(first, last):
        for li, (spec, ring, p0, xs) in enumerate(layers):
            kc, vc, ws, desc, _ = state[li]
            x = xs[s]
            pos = torch.from_numpy((p0 + s).astype(np.int32)).cuda()
            mp = int((p0 + s).max())
            o = hswd.layer_step(x["q"], x["k"], x["v"], x["gate"], kc, vc, pos, ring, spec.rot,
                                spec.theta, ws, max_pos=mp, desc=desc)
            outs[(s, li)] = _bits(o).clone()
    torch.cuda.synchronize()
    return outs


def _fresh_state(layers, caches):
    state = []
    for (spec, ring, p0, xs), (kc, vc) in zip(layers, caches):
        # the descriptor keeps a raw pointer to the scales: the tensor lives
        # in the state beside it
        sc = None if spec.kv_scale is None else torch.from_numpy(spec.kv_scale).cuda()
        desc = hswd.make_desc(kc, n_heads=spec.H, kv_scale=sc)
        mp = int(p0.max()) + 16
        state.append((kc, vc, hswd.workspace(desc, ring, mp), desc, sc))
    return state


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_checkpoint_and_resume_equal_an_uninterrupted_run(dtype):
    steps, cut = 12, 5
    B = 4
    p0 = np.array([505, 509, 2, 1000], np.int64)       # two rings wrap during the run
    rng = np.random.default_rng(90)
    layers = []
    for kind in ("sliding", "full"):
        spec = (inputs.sliding_spec(B, dtype) if kind == "sliding"
                else inputs.full_spec(B, int(p0.max()) + steps + 1, dtype))
        xs = [{n: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda()
               for n, shape in (("q", (B, spec.H, spec.D)), ("k", (B, spec.Hkv, spec.D)),
                                ("v", (B, spec.Hkv, spec.D)), ("gate", (B, spec.H)))}
              for _ in range(steps)]
        layers.append((spec, kind == "sliding", p0, xs))
    init = [inputs.device_step(spec, p0, seed=91 + i, device="cuda")
            for i, (spec, _, _, _) in enumerate(layers)]
    say("resume: %s, %d steps, cut after step %d" % (dtype, steps, cut))

    # uninterrupted
    a_caches = [(t["k_cache"].clone(), t["v_cache"].clone()) for t in init]
    a_state = _fresh_state(layers, a_caches)
    a_out = _run_steps(layers, steps, 0, steps, a_state)

    # interrupted after `cut` steps: caches to the host, then into fresh buffers
    b_caches = [(t["k_cache"].clone(), t["v_cache"].clone()) for t in init]
    b_state = _fresh_state(layers, b_caches)
    b_out = _run_steps(layers, steps, 0, cut, b_state)
    snap = [(_bits(kc).cpu().numpy().copy(), _bits(vc).cpu().numpy().copy())
            for kc, vc, _, _, _ in b_state]
    del b_state, b_caches
    torch.cuda.synchronize()
    restored = []
    for (kb, vb), t in zip(snap, init):
        kc = torch.empty_like(t["k_cache"])
        vc = torch.empty_like(t["v_cache"])
        _bits(kc).copy_(torch.from_numpy(kb))
        _bits(vc).copy_(torch.from_numpy(vb))
        restored.append((kc, vc))
    r_state = _fresh_state(layers, restored)
    b_out.update(_run_steps(layers, steps, cut, steps, r_state))

    for key in a_out:
        assert torch.equal(a_out[key], b_out[key]), key
    for (akc, avc, _, _, _), (rkc, rvc, _, _, _) in zip(a_state, r_state):
        assert torch.equal(_bits(akc), _bits(rkc))
        assert torch.equal(_bits(avc), _bits(rvc))
