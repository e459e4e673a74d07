"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one hswd_layer_step per layer, default chunking).

Every (stream, query head) is checked: the fp64 oracle runs the whole layer
step on host copies of the same device data (OpenMP over (stream, head)) and
each head's output is compared under the parity bar, normalised per (stream,
kv head) by the largest attended |V|.  The stored entries are checked bit for
bit for every (stream, kv head), and every other cache row must be untouched
(compared on the device with a copy taken before the step)."""
import time

import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import CODE, TOL, cache_to_host, entry_codes, say

pytestmark = pytest.mark.gpu


def _bits(t):
    """Integer view of a cache tensor, so NaN poison compares equal to itself."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def _host_rows(cache, bidx, rows):
    """Host bits of row rows[b] of every (stream b, kv head), [B, Hkv, D], in
    the oracle's storage type (uint8 codes, uint16 bits or float32)."""
    a = _bits(cache)[bidx, :, rows].cpu().numpy()
    return {1: lambda x: x, 2: lambda x: x.view(np.uint16),
            4: lambda x: x.view(np.float32)}[cache.element_size()](a)


def vmax_per_pair(vc_host, code, pos, n_slots, v, vscale):
    """max |V| over the rows each (stream, kv head) attends plus the new v,
    decoded one block at a time (a whole long cache in float64 would not fit
    comfortably in host memory)."""
    B, Hkv = vc_host.shape[:2]
    out = np.zeros((B, Hkv))
    for b in range(B):
        n = min(max(int(pos[b]), 0), n_slots)
        for g in range(Hkv):
            m = float(np.abs(oracle.decode(code, vc_host[b, g, :n])).max()) * vscale[g] if n else 0.0
            out[b, g] = max(m, float(np.abs(v[b, g]).max()))
    return out


def check_layer(spec, pos, seed):
    dev = torch.device("cuda", 0)
    ring = spec.kind == "sliding"
    code = CODE[spec.dtype]
    G = spec.H // spec.Hkv
    t = inputs.device_step(spec, pos, seed=seed, device=dev)
    B, S = spec.B, spec.n_slots
    mp = int(t["pos"].max())
    desc = hswd.make_desc(t["k_cache"], n_heads=spec.H, kv_scale=t.get("kv_scale"))
    ws = hswd.workspace(desc, ring, mp)
    ks = spec.kv_scale[0] if spec.kv_scale is not None else np.ones(spec.Hkv, np.float32)
    vs = spec.kv_scale[1] if spec.kv_scale is not None else np.ones(spec.Hkv, np.float32)
    kc_host = cache_to_host(t["k_cache"])          # before the step writes its entry
    vc_host = cache_to_host(t["v_cache"])
    k_before = t["k_cache"].clone()
    v_before = t["v_cache"].clone()
    q, k, v, gate = (t[x].cpu().numpy() for x in ("q", "k", "v", "gate"))
    posh = t["pos"].cpu().numpy()
    say("full-size %s %s B=%d H=%d Hkv=%d pos=%s..., every (stream, head)" % (
        spec.kind, spec.dtype, B, spec.H, spec.Hkv, list(posh[:4])))
    out = hswd.layer_step(t["q"], t["k"], t["v"], t["gate"], t["k_cache"], t["v_cache"], t["pos"],
                          ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
    assert hswd.check_errors(ws) == 0
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))

    t0 = time.time()
    r = oracle.layer_step(q, k, v, gate, kc_host, vc_host, posh, code, ring, spec.rot, spec.theta,
                          write=False, kv_scale=spec.kv_scale)
    assert r["status"] == 0
    say("  oracle over %d (stream, head): %.1f s" % (B * spec.H, time.time() - t0))
    vmax = vmax_per_pair(vc_host, code, posh, S, v, vs)
    err = np.abs(out - r["out"]).max(axis=2) / np.repeat(vmax, G, axis=1)
    worst = float(err.max())
    b, h = np.unravel_index(int(err.argmax()), err.shape)
    say("  worst normalised error %.3e at (stream %d, head %d), bar %.0e" % (
        worst, b, h, TOL[spec.dtype]))
    assert worst <= TOL[spec.dtype], (worst, b, h)

    # stored entries, bit for bit: v from the oracle's rounding, k given the
    # GPU's float32 rotated key (both sides round an fp64 rotation once to
    # float32; the codes are checked from the same float32 input)
    kr = t["k"].clone()
    hswd.rope_apply(torch.zeros_like(t["q"]), kr, t["pos"], spec.rot, spec.theta)
    kr = kr.cpu().numpy()
    rows = torch.as_tensor([(p % S) if ring else p for p in posh], dtype=torch.long, device=dev)
    bidx = torch.arange(B, device=dev)
    k_new = _host_rows(t["k_cache"], bidx, rows)          # [B, Hkv, D]
    v_new = _host_rows(t["v_cache"], bidx, rows)
    for g in range(spec.Hkv):
        sk = None if spec.kv_scale is None else ks[g]
        assert np.array_equal(k_new[:, g], entry_codes(kr[:, g], spec.dtype, sk)), g
    assert np.array_equal(v_new, r["v_hat"])
    # every other row untouched
    _bits(k_before)[bidx, :, rows] = _bits(t["k_cache"])[bidx, :, rows]
    _bits(v_before)[bidx, :, rows] = _bits(t["v_cache"])[bidx, :, rows]
    assert torch.equal(_bits(k_before), _bits(t["k_cache"]))
    assert torch.equal(_bits(v_before), _bits(t["v_cache"]))
    del t, k_before, v_before
    torch.cuda.empty_cache()


def test_step_layers_64x4096():
    """A sliding and a full layer of the 28-layer step: 64 streams at 4096,
    all 512 (stream, head) of each."""
    check_layer(inputs.sliding_spec(64, "bf16"), 4096, 4000)
    check_layer(inputs.full_spec(64, 4097, "bf16"), 4096, 4003)


def test_long_context_8x131072():
    """8 streams at context 131072: full layer (128 chunks of 1024 keys, several
    workgroups per (stream, head), last-arrival merge) and a sliding layer
    at the same positions; all 64 (stream, head) of each."""
    check_layer(inputs.full_spec(8, 131073, "bf16"), 131072, 5000)
    check_layer(inputs.sliding_spec(8, "bf16"), 131072, 5001)


def test_long_context_grouped_fp8_8x131072():
    """8 streams at context 131072, 32 query heads over 8 kv heads, fp8
    cache: the 4-head matrix-core kernel over 128 chunks of 1024 keys,
    merged across workgroups; all 256 (stream, head)."""
    check_layer(inputs.full_spec(8, 131073, "fp8", H=32), 131072, 5200)


def test_ragged_long_context_packed_split():
    """8 streams of a 131073-row cache at ragged positions (from empty to the
    capacity, a stream far below it, one past 32768 keys only): the packed
    split deals the launch's workgroups out by valid keys, so the streams
    get different workgroup counts and chunk sizes; all 64 (stream, head),
    bf16, and again over fp8 with 32 query heads (the 4-head kernel)."""
    pos = np.array([131072, 0, 5000, 40000, 33000, 90000, 1, 70001], np.int64)
    check_layer(inputs.full_spec(8, 131073, "bf16"), pos, 5300)
    check_layer(inputs.full_spec(8, 131073, "fp8", H=32), pos[::-1].copy(), 5301)


def test_packed_split_more_streams_than_slots():
    """72 streams over 8 kv heads (more (stream, kv head) pairs than the GPU
    holds workgroups at once) at ragged positions up to 33000 keys, fp8,
    128 dims: the packed deal then bounds the launch's workgroups by its
    pack plus one per pair and still gives the longest streams several;
    all 576 (stream, head)."""
    pos = inputs.ragged_positions(72, 0, 33000, seed=5400)
    pos[0] = 33000
    check_layer(inputs.full_spec(72, 33001, "fp8", D=128), pos, 5401)


def test_ragged_full_layer_64_streams():
    """64 streams with ragged positions in [1, 4096] on a full layer: most
    chunks of the short streams are empty."""
    pos = inputs.ragged_positions(64, 1, 4096, seed=6)
    check_layer(inputs.full_spec(64, 4097, "bf16"), pos, 4010)


def test_ragged_sliding_layer_64_streams():
    """The batched sliding layer: 64 rings with ragged positions in [1, 4096],
    some partly filled."""
    pos = inputs.ragged_positions(64, 1, 4096, seed=3)
    check_layer(inputs.sliding_spec(64, "bf16"), pos, 4011)


def test_step_layers_64x4096_fp8():
    """The fp8 step's layers (per-head scales): 64 streams at 4096."""
    check_layer(inputs.sliding_spec(64, "fp8"), 4096, 4100)
    check_layer(inputs.full_spec(64, 4097, "fp8"), 4096, 4103)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_grouped_step_layers_64x4096(dtype):
    """The grouped step's layers: 32 query heads over 8 kv heads (4 per kv
    head), 64 streams at 4096; all 2048 (stream, head)."""
    check_layer(inputs.sliding_spec(64, dtype, H=32), 4096, 4200)
    check_layer(inputs.full_spec(64, 4097, dtype, H=32), 4096, 4203)


def test_grouped_step_layers_64x4096_h64():
    """64 query heads over 8 kv heads: the 8-head kernel (one workgroup
    per group, the value product on the matrix cores), bf16 and fp8."""
    check_layer(inputs.full_spec(64, 4097, "bf16", H=64), 4096, 4300)
    check_layer(inputs.full_spec(64, 4097, "fp8", H=64), 4096, 4301)


def test_very_long_stream_four_kv_heads():
    """One stream at 2^19 + 1000 keys over 4 kv heads (128 dims): past the
    2^19-key tier its chunk is 4096 keys (1024 per kv head), so the lone
    stream still spreads over 512 chunks; every head."""
    check_layer(inputs.full_spec(1, (1 << 19) + 1001, "bf16", H=4, Hkv=4, D=128),
                (1 << 19) + 1000, 5500)


def test_max_context_1x1048576():
    """One stream at context 2^20 on a full layer (8.6 GB of cache, 128
    chunks of 8192 keys, 64 workgroups per kv head merged by the last to
    arrive): the largest context the tests exercise; all 8 heads."""
    check_layer(inputs.full_spec(1, (1 << 20) + 1, "bf16"), 1 << 20, 5100)
