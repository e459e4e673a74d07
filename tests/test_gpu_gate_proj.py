"""GPU parity of the gate projection (g_proj: hidden 2048 -> one logit per
head), standalone and fused into the layer step."""
import numpy as np
import pytest

import hybrid_sliding_window_decode_amd as hswd
import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import CODE, assert_parity, f32_dev, say, to_dev

pytestmark = pytest.mark.gpu


def test_gate_proj_matches_oracle():
    x, w = inputs.gate_inputs(64, 2048, 8, seed=60)
    say("gate_proj 64x2048x8")
    got = hswd.gate_proj(f32_dev(x), f32_dev(w)).cpu().numpy()
    ref = oracle.gate_proj(x, w)
    scale = np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T   # sum of |terms|
    assert np.all(np.abs(got - ref) <= 1e-6 * scale)
    x2, w2 = inputs.gate_inputs(3, 1000, 5, seed=61)                       # ragged sizes
    got2 = hswd.gate_proj(f32_dev(x2), f32_dev(w2)).cpu().numpy()
    ref2 = oracle.gate_proj(x2, w2)
    assert np.all(np.abs(got2 - ref2) <= 1e-6 * (np.abs(x2) @ np.abs(w2).T))


@pytest.mark.parametrize("kind,dtype,G", [("sliding", "bf16", 1), ("full", "f16", 1),
                                          ("sliding", "bf16", 4), ("full", "bf16", 2),
                                          ("full", "bf16", 8), ("sliding", "fp8", 8)])
def test_layer_step_gproj(kind, dtype, G):
    """Fused projection + step: the same bits as gate_proj then layer_step,
    and the oracle's output scaled by the oracle's sigmoid(logit); G query
    heads per kv head (each head keeps its own row of w_g)."""
    B = 12
    ring = kind == "sliding"
    Hkv = 8 // G
    spec = (inputs.sliding_spec(B, dtype, Hkv=Hkv) if ring
            else inputs.full_spec(B, 3000, dtype, Hkv=Hkv))
    pos = inputs.ragged_positions(B, 0, 4096 if ring else 2999, seed=62)
    x = inputs.make_step(spec, pos, seed=63)
    gx, gw = inputs.gate_inputs(B, 2048, 8, seed=64)
    mp = int(x.pos.max())
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"], n_heads=8, kv_scale=d["kv_scale"])
    ws = hswd.workspace(desc, ring, mp)
    say("layer_step_gproj %s %s G=%d" % (kind, dtype, G))
    fused = hswd.layer_step_gproj(d["q"], d["k"], d["v"], f32_dev(gx), f32_dev(gw), d["k_cache"],
                                  d["v_cache"], d["pos"], ring, spec.rot, spec.theta, ws,
                                  max_pos=mp, desc=desc).cpu().numpy()
    e = to_dev(x)
    logits = hswd.gate_proj(f32_dev(gx), f32_dev(gw))
    two = hswd.layer_step(e["q"], e["k"], e["v"], logits, e["k_cache"], e["v_cache"], e["pos"],
                          ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc).cpu().numpy()
    assert hswd.check_errors(ws) == 0
    assert np.array_equal(fused, two)
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    r = oracle.layer_step(x.q, x.k, x.v, None, kc, vc, x.pos, CODE[dtype], ring, spec.rot,
                          spec.theta, write=False, kv_scale=spec.kv_scale)
    lg = oracle.gate_proj(gx, gw)
    ref = r["o_pre"] * (1.0 / (1.0 + np.exp(-lg)))[:, :, None]
    assert_parity(fused, ref, x, "gproj step")
