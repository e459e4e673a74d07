"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one hswd_layer_step per layer, default chunking): the
oracle recomputes sampled (stream, head) outputs one by one from host copies
of the same device data; the stored entries are checked bit for bit."""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import TOL, cache_to_host, say

pytestmark = pytest.mark.gpu

BF16 = oracle.BF16


def check_layer(spec, pos, seed, samples):
    dev = torch.device("cuda", 0)
    ring = spec.kind == "sliding"
    t = inputs.device_step(spec, pos, seed=seed, device=dev)
    B = spec.B
    mp = int(t["pos"].max())
    desc = hswd.make_desc(t["k_cache"])
    ws = hswd.workspace(desc, ring, mp)
    # host copies of the sampled blocks before the step writes its entry
    blocks = {}
    for b, h in samples:
        blocks[(b, h)] = (cache_to_host(t["k_cache"][b, h]), cache_to_host(t["v_cache"][b, h]))
    q, k, v, gate = (t[x].cpu().numpy() for x in ("q", "k", "v", "gate"))
    posh = t["pos"].cpu().numpy()
    say("full-size %s B=%d pos=%s, %d samples" % (spec.kind, B, list(posh[:4]), len(samples)))
    out = hswd.layer_step(t["q"], t["k"], t["v"], t["gate"], t["k_cache"], t["v_cache"], t["pos"],
                          ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
    assert hswd.check_errors(ws) == 0
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    # the GPU's rotated key (same device RoPE as the fused step) for the entry check
    kr = t["k"].clone()
    hswd.rope_apply(torch.zeros_like(t["q"]), kr, t["pos"], spec.rot, spec.theta)
    kr = kr.cpu().numpy()
    worst = 0.0
    for (b, h), (kc, vc) in blocks.items():
        p = int(posh[b])
        n = min(p, spec.n_slots)
        q_rot = oracle.rope(q[b, h][None, None], [p], spec.rot, spec.theta)[0, 0]
        k_rot = oracle.rope(k[b, h][None, None], [p], spec.rot, spec.theta)[0, 0]
        k_hat = oracle.round_to(BF16, k_rot.astype(np.float32))
        v_hat = oracle.round_to(BF16, v[b, h])
        o = oracle.attend_block(q_rot, kc, vc, BF16, n, k_hat, v_hat, 1.0 / np.sqrt(spec.D))
        ref = o * oracle.sigmoid(float(gate[b, h]))
        vd = oracle.decode(BF16, vc[:n])
        vmax = max(float(np.abs(vd).max()) if n else 0.0, float(np.abs(v[b, h]).max()))
        err = float(np.max(np.abs(out[b, h] - ref)) / vmax)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, h, err)
        # the stored entry, bit for bit, given the GPU's float32 rotated key
        row = p % spec.n_slots if ring else p
        assert np.array_equal(cache_to_host(t["k_cache"][b, h, row]),
                              oracle.round_to(BF16, kr[b, h]))
        assert np.array_equal(cache_to_host(t["v_cache"][b, h, row]), v_hat)
    say("  worst normalised error %.3e over %d sampled (stream, head)" % (worst, len(blocks)))
    del t
    torch.cuda.empty_cache()


def samples(B, H, n, seed):
    rng = np.random.default_rng(seed)
    s = {(0, 0), (B - 1, H - 1)}
    while len(s) < n:
        s.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(s)


def test_step_layers_64x4096():
    """A sliding and a full layer of the 28-layer step: 64 streams at 4096."""
    check_layer(inputs.sliding_spec(64, "bf16"), 4096, 4000, samples(64, 8, 24, 1))
    check_layer(inputs.full_spec(64, 4097, "bf16"), 4096, 4003, samples(64, 8, 24, 2))


def test_long_context_8x131072():
    """8 streams at context 131072: full layer (256 chunks, several
    workgroups per (stream, head), last-arrival merge) and a sliding layer
    at the same positions."""
    check_layer(inputs.full_spec(8, 131073, "bf16"), 131072, 5000, samples(8, 8, 8, 3))
    check_layer(inputs.sliding_spec(8, "bf16"), 131072, 5001, samples(8, 8, 16, 4))


def test_ragged_full_layer_64_streams():
    """64 streams with ragged positions in [1, 4096] on a full layer: most
    chunks of the short streams are empty."""
    pos = inputs.ragged_positions(64, 1, 4096, seed=6)
    check_layer(inputs.full_spec(64, 4097, "bf16"), pos, 4010, samples(64, 8, 24, 5))
