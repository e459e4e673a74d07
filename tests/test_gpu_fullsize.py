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
from gpu_util import CODE, TOL, cache_to_host, entry_codes, say

pytestmark = pytest.mark.gpu

def check_layer(spec, pos, seed, samples):
    """samples: (stream, query head) pairs; query head h reads kv head h // G."""
    dev = torch.device("cuda", 0)
    ring = spec.kind == "sliding"
    code = CODE[spec.dtype]
    G = spec.H // spec.Hkv
    t = inputs.device_step(spec, pos, seed=seed, device=dev)
    B = spec.B
    mp = int(t["pos"].max())
    desc = hswd.make_desc(t["k_cache"], n_heads=spec.H, kv_scale=t.get("kv_scale"))
    ws = hswd.workspace(desc, ring, mp)
    ks = spec.kv_scale[0] if spec.kv_scale is not None else np.ones(spec.Hkv)
    vs = spec.kv_scale[1] if spec.kv_scale is not None else np.ones(spec.Hkv)
    # host copies of the sampled blocks before the step writes its entry
    blocks = {}
    for b, h in samples:
        g = h // G
        if (b, g) not in blocks:
            blocks[(b, g)] = (cache_to_host(t["k_cache"][b, g]), cache_to_host(t["v_cache"][b, g]))
    q, k, v, gate = (t[x].cpu().numpy() for x in ("q", "k", "v", "gate"))
    posh = t["pos"].cpu().numpy()
    say("full-size %s %s B=%d H=%d Hkv=%d pos=%s, %d samples" % (
        spec.kind, spec.dtype, B, spec.H, spec.Hkv, list(posh[:4]), len(samples)))
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
    for b, h in samples:
        g = h // G
        kc, vc = blocks[(b, g)]
        p = int(posh[b])
        n = min(p, spec.n_slots)
        q_rot = oracle.rope(q[b, h][None, None], [p], spec.rot, spec.theta)[0, 0]
        k_rot = oracle.rope(k[b, g][None, None], [p], spec.rot, spec.theta)[0, 0]
        k_hat = entry_codes(k_rot.astype(np.float32), spec.dtype,
                            None if spec.kv_scale is None else ks[g])
        v_hat = entry_codes(v[b, g], spec.dtype, None if spec.kv_scale is None else vs[g])
        o = oracle.attend_block(q_rot, kc, vc, code, n, k_hat, v_hat, 1.0 / np.sqrt(spec.D),
                                float(ks[g]), float(vs[g]))
        ref = o * oracle.sigmoid(float(gate[b, h]))
        vd = oracle.decode(code, vc[:n]) * float(vs[g])
        vmax = max(float(np.abs(vd).max()) if n else 0.0, float(np.abs(v[b, g]).max()))
        err = float(np.max(np.abs(out[b, h] - ref)) / vmax)
        worst = max(worst, err)
        assert err <= TOL[spec.dtype], (b, h, err)
        # the stored entry, bit for bit, given the GPU's float32 rotated key
        row = p % spec.n_slots if ring else p
        assert np.array_equal(cache_to_host(t["k_cache"][b, g, row]),
                              entry_codes(kr[b, g], spec.dtype,
                                          None if spec.kv_scale is None else ks[g]))
        assert np.array_equal(cache_to_host(t["v_cache"][b, g, row]), v_hat)
    say("  worst normalised error %.3e over %d sampled (stream, head)" % (worst, len(samples)))
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
    """8 streams at context 131072: full layer (128 chunks of 1024 keys, several
    workgroups per (stream, head), last-arrival merge) and a sliding layer
    at the same positions."""
    check_layer(inputs.full_spec(8, 131073, "bf16"), 131072, 5000, samples(8, 8, 8, 3))
    check_layer(inputs.sliding_spec(8, "bf16"), 131072, 5001, samples(8, 8, 16, 4))


def test_long_context_grouped_fp8_8x131072():
    """8 streams at context 131072, 32 query heads over 8 kv heads, fp8
    cache: the 4-head matrix-core kernel over 128 chunks of 1024 keys,
    merged across workgroups."""
    check_layer(inputs.full_spec(8, 131073, "fp8", H=32), 131072, 5200, samples(8, 32, 12, 12))


def test_ragged_full_layer_64_streams():
    """64 streams with ragged positions in [1, 4096] on a full layer: most
    chunks of the short streams are empty."""
    pos = inputs.ragged_positions(64, 1, 4096, seed=6)
    check_layer(inputs.full_spec(64, 4097, "bf16"), pos, 4010, samples(64, 8, 24, 5))


def test_step_layers_64x4096_fp8():
    """The fp8 step's layers (per-head scales): 64 streams at 4096."""
    check_layer(inputs.sliding_spec(64, "fp8"), 4096, 4100, samples(64, 8, 16, 7))
    check_layer(inputs.full_spec(64, 4097, "fp8"), 4096, 4103, samples(64, 8, 16, 8))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_grouped_step_layers_64x4096(dtype):
    """The grouped step's layers: 32 query heads over 8 kv heads (4 per kv
    head), 64 streams at 4096."""
    check_layer(inputs.sliding_spec(64, dtype, H=32), 4096, 4200, samples(64, 32, 16, 9))
    check_layer(inputs.full_spec(64, 4097, dtype, H=32), 4096, 4203, samples(64, 32, 16, 10))


def test_max_context_1x1048576():
    """One stream at context 2^20 on a full layer (8.6 GB of cache, 512
    chunks of 2048 keys, 64 workgroups per kv head merged by the last to
    arrive): the largest context the tests exercise."""
    check_layer(inputs.full_spec(1, (1 << 20) + 1, "bf16"), 1 << 20, 5100, samples(1, 8, 8, 11))
