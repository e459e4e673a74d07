"""GPU parity of the per-token kernels: slot/mask, RoPE, entry write, head
gate and split merge, each through the C ABI against the oracle."""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
import oracle
import pins
from gpu_util import (CODE, cache_to_dev, cache_to_host, entry_codes, f32_dev, i32_dev, say,
                      to_dev)
from hybrid_sliding_window_decode_amd import inputs

pytestmark = pytest.mark.gpu

POS = np.array([0, 1, 2, 89, 510, 511, 512, 600, 1021, 1022, 1023, 4095, 4096, 131072],
               np.int32)


@pytest.mark.parametrize("ring", [1, 0])
def test_ring_mask_bit_exact(ring):
    S = 511 if ring else 131073
    say("ring_mask ring=%d S=%d" % (ring, S))
    mask, slot = hswd.ring_mask(i32_dev(POS), S, ring)
    om_slot, om_mask = oracle.slot_mask(POS, S, ring)
    assert np.array_equal(slot.cpu().numpy(), om_slot)
    assert np.array_equal(mask.cpu().numpy(), om_mask)


@pytest.mark.parametrize("rot,theta,H", [(256, 1e4, 8), (64, 5e6, 8), (128, 1e4, 8),
                                         (256, 1e4, 64)])
def test_rope(rot, theta, H):
    rng = np.random.default_rng(40 + rot)
    B, Hkv, D = len(POS), 8, 256
    q = rng.standard_normal((B, H, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    say("rope rot=%d theta=%g B=%d" % (rot, theta, B))
    qd, kd = f32_dev(q), f32_dev(k)
    hswd.rope_apply(qd, kd, i32_dev(POS), rot, theta)
    gq, gk = qd.cpu().numpy(), kd.cpu().numpy()
    for got, x, nh in [(gq, q, H), (gk, k, Hkv)]:
        ref = oracle.rope(x, POS, rot, theta)
        # the GPU rounds its double-precision rotation once to float32
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp), np.max(np.abs(got - ref) / ulp)
        assert np.array_equal(got[0], x[0])                    # pos 0: identity
        assert np.array_equal(got[..., rot:], x[..., rot:])    # untouched dims


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
def test_kv_slot_write_rounding_bit_exact(dtype):
    """Entry rounding on the GPU equals the oracle's, bit for bit, on 2^24
    random float32 patterns and on every tie and edge of the target grid
    (fp8: of x / scale with a different scale per kv head)."""
    rng = np.random.default_rng(41)
    special = pins.fp8_special_inputs() if dtype == "fp8" else pins.rne_special_inputs()
    vals = np.concatenate([
        rng.integers(0, 2 ** 32, size=1 << 24, dtype=np.uint64).astype(np.uint32).view(np.float32),
        special])
    Hkv, D = 8, 256
    per = Hkv * D
    B = -(-vals.size // per)
    vals = np.resize(vals, B * per).astype(np.float32)
    k = vals.reshape(B, Hkv, D)
    v = np.roll(vals, 12345).reshape(B, Hkv, D)
    sd = oracle.storage_dtype(CODE[dtype])
    kc = np.zeros((B, Hkv, 3, D), sd)
    say("kv_slot_write %s B=%d" % (dtype, B))
    kd, vd = cache_to_dev(kc, dtype), cache_to_dev(kc.copy(), dtype)
    pos = np.arange(B, dtype=np.int32)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    slot = torch.empty(B, dtype=torch.int32, device="cuda")
    sc = inputs.default_fp8_scales(Hkv) if dtype == "fp8" else None
    sc_dev = None if sc is None else f32_dev(sc)
    desc = hswd.make_desc(kd, kv_scale=sc_dev)
    hswd.kv_slot_write(kd, vd, f32_dev(k), f32_dev(v), i32_dev(pos), 1, ws, slot_out=slot,
                       desc=desc)
    assert hswd.check_errors(ws) == 0
    kh, vh = cache_to_host(kd), cache_to_host(vd)
    assert np.array_equal(slot.cpu().numpy(), pos % 3)
    for b in range(0, B, 97):
        assert np.all(kh[b, :, [s for s in range(3) if s != b % 3]] == 0)
    ref_k = entry_codes(k, dtype, None if sc is None else sc[0][None, :, None])
    ref_v = entry_codes(v, dtype, None if sc is None else sc[1][None, :, None])
    rows = pos % 3
    got_k = kh[np.arange(B), :, rows]
    got_v = vh[np.arange(B), :, rows]
    if dtype == "f32":
        assert np.array_equal(got_k.view(np.uint32), ref_k.view(np.uint32))
        assert np.array_equal(got_v.view(np.uint32), ref_v.view(np.uint32))
    else:
        assert np.array_equal(got_k, ref_k)
        assert np.array_equal(got_v, ref_v)


@pytest.mark.parametrize("H", [8, 32, 64])
def test_fp8_decode_all_codes_in_attention(H):
    """A one-key cache holding each of the 255 non-NaN fp8 codes in turn
    (q = 0, new value 0): the output is the mean of the decoded cached value
    and 0 -- the kernel's fp8 decode of every code, against the oracle's
    (H = 32, 64: the 4- and 8-head kernels' value paths)."""
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)
    B, D = len(codes), 256
    spec = inputs.sliding_spec(B, "fp8", n_slots=511, H=H)
    x = inputs.make_step(spec, 1, seed=45)
    x.q[:] = 0
    x.v[:] = 0
    x.k[:] = 0
    x.v_cache[:, :, 0, :] = codes[:, None, None]
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"], n_heads=H, kv_scale=d["kv_scale"])
    ws = hswd.workspace(desc, 1, 0)
    say("fp8 decode of all codes, H=%d" % H)
    hswd.rope_apply(d["q"], d["k"], d["pos"], 256, 1e4)
    o = hswd.decode_attn_sliding(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["pos"],
                                 ws, desc=desc).cpu().numpy()
    val = oracle.decode(CODE["fp8"], codes)[:, None] * spec.kv_scale[1][None, :]
    G = H // 8
    assert np.array_equal(o[:, :, 0].astype(np.float64), np.repeat(val, G, axis=1) / 2)


@pytest.mark.parametrize("H", [8, 32, 64])
def test_fp8_key_decode_all_codes_in_attention(H):
    """A one-key cache whose key holds one of the 255 non-NaN fp8 codes in
    every dim, value 1; new key and value 0; the query a multiple t of the
    first unit vector, t chosen so the cached score is about 1: the output's
    first dim is sigmoid(score), so a mis-decoded key code moves it far
    beyond the bar.  Against the oracle, all codes, both kernels."""
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)
    B, D = len(codes), 256
    spec = inputs.sliding_spec(B, "fp8", n_slots=511, H=H)
    x = inputs.make_step(spec, 1, seed=46)
    dec = oracle.decode(CODE["fp8"], codes)
    ks = spec.kv_scale[0]
    t = np.where(dec == 0, 1.0, 16.0 / np.where(dec == 0, 1.0, np.abs(dec)))
    x.q[:] = 0
    x.q[:, :, 0] = (t[:, None] / ks[np.arange(H) // (H // 8)][None, :]).astype(np.float32)
    x.k[:] = 0
    x.v[:] = 0
    x.k_cache[:, :, 0, :] = codes[:, None, None]
    x.v_cache[:, :, 0, :] = 0x38                      # 1.0
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"], n_heads=H, kv_scale=d["kv_scale"])
    ws = hswd.workspace(desc, 1, 0)
    say("fp8 key decode of all codes, H=%d" % H)
    o = hswd.decode_attn_sliding(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["pos"],
                                 ws, desc=desc).cpu().numpy()
    # the oracle's attention of the same rotated query (no rotation here)
    want = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            g = h // (H // 8)
            kc = x.k_cache[b, g, :1]
            vc = x.v_cache[b, g, :1]
            kh = np.zeros(D, np.uint8)
            want[b, h] = oracle.attend_block(x.q[b, h].astype(np.float64), kc, vc, CODE["fp8"],
                                             1, kh, kh, 1 / 16.0, ks=float(ks[g]),
                                             vs=float(spec.kv_scale[1][g]))[0]
    vs = np.repeat(spec.kv_scale[1], H // 8)[None, :]
    assert np.max(np.abs(o[:, :, 0] - want) / vs) <= 2e-3


def test_kv_slot_write_capacity_flag():
    B, Hkv, S, D = 4, 8, 10, 256
    rng = np.random.default_rng(42)
    k = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    pos = np.array([3, 10, 9, 11], np.int32)       # 10 and 11 do not fit 10 rows
    kc = torch.zeros(B, Hkv, S, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    slot = torch.empty(B, dtype=torch.int32, device="cuda")
    say("kv_slot_write capacity")
    hswd.kv_slot_write(kc, vc, f32_dev(k), f32_dev(k), i32_dev(pos), 0, ws, slot_out=slot)
    assert hswd.check_errors(ws) == hswd.binding.FLAG_CAPACITY
    assert slot.cpu().tolist() == [3, -1, 9, -1]
    assert float(kc[1].abs().sum()) == 0 and float(kc[3].abs().sum()) == 0
    hswd.workspace_init(ws)
    assert hswd.check_errors(ws) == 0


def test_head_gate():
    rng = np.random.default_rng(43)
    B, H, D = 64, 8, 256
    o = rng.standard_normal((B, H, D), dtype=np.float32)
    g = rng.standard_normal((B, H), dtype=np.float32) * 4
    g[0, :4] = [0, 40, -40, 88]
    say("head_gate")
    got = hswd.head_gate(f32_dev(o), f32_dev(g)).cpu().numpy()
    ref = oracle.head_gate(o.astype(np.float64), g)
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)) < 2e-6
    assert np.array_equal(got[0, 0], o[0, 0] * np.float32(0.5))
    # in place
    od = f32_dev(o)
    hswd.head_gate(od, f32_dev(g), out=od)
    assert np.array_equal(od.cpu().numpy(), got)


@pytest.mark.parametrize("n", [1, 7, 16, 40, 256])
def test_lse_merge(n):
    rng = np.random.default_rng(44 + n)
    B, H, D = 3, 8, 256
    m = rng.standard_normal((B, H, n)).astype(np.float32) * 3
    l = rng.uniform(0.5, 50, (B, H, n)).astype(np.float32)
    o = (rng.standard_normal((B, H, n, D)) * 5).astype(np.float32)
    if n > 1:                                      # empty partials are skipped
        m[:, :, ::3] = -np.inf
        l[:, :, ::3] = 0
        o[:, :, ::3] = 0
    ml = np.stack([m, l], -1)
    say("lse_merge n=%d" % n)
    got = hswd.lse_merge(f32_dev(o), f32_dev(ml)).cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = oracle.merge(m[b, h], l[b, h], o[b, h])
            err = np.max(np.abs(got[b, h] - ref)) / np.max(np.abs(ref))
            assert err < 1e-5, (b, h, err)


def test_stream_read_helper():
    """The measurement helper reads a buffer and leaves its sink untouched."""
    import torch
    say("stream_read 64 MiB")
    buf = torch.arange(1 << 24, dtype=torch.int32, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    for wgs in (1, 7, 512):
        hswd.stream_read(buf, wgs, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_empty_batch_through_the_binding():
    """Zero streams: every entry accepts the empty tensors, launches nothing
    and returns empty outputs."""
    say("empty batch")
    dev = "cuda"
    q = torch.empty(0, 8, 256, device=dev)
    k = torch.empty(0, 8, 256, device=dev)
    v = torch.empty(0, 8, 256, device=dev)
    gate = torch.empty(0, 8, device=dev)
    pos = torch.empty(0, dtype=torch.int32, device=dev)
    kc = torch.empty(0, 8, 511, 256, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    desc = hswd.make_desc(kc)
    ws = hswd.workspace(desc, 1, 0)
    hswd.rope_apply(q, k, pos, 256, 1e4)
    o = hswd.decode_attn_sliding(q, k, v, kc, vc, pos, ws, desc=desc)
    assert tuple(o.shape) == (0, 8, 256)
    g = hswd.head_gate(o, gate)
    hswd.kv_slot_write(kc, vc, k, v, pos, 1, ws, desc=desc)
    out = hswd.layer_step(q, k, v, gate, kc, vc, pos, 1, 256, 1e4, ws, desc=desc)
    mask, slot = hswd.ring_mask(pos, 511, 1)
    torch.cuda.synchronize()
    assert hswd.check_errors(ws) == 0
    assert out.numel() == 0 and g.numel() == 0 and slot.numel() == 0 and mask.numel() == 0
