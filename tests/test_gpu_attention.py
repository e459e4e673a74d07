"""GPU parity of the decode attention entry points against the oracle, at
sizes the oracle finishes in seconds that still span several tiles, several
splits and ragged tails, plus the method's degenerate cases."""
import math
import zlib

import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
import oracle
from oracle import brute
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import (CODE, assert_parity, cache_to_dev, cache_to_host, entry_codes, f32_dev,
                      i32_dev, say, to_dev)

pytestmark = pytest.mark.gpu


def spec_for(kind, B, dtype, S=None, H=8, D=256):
    if kind == "sliding":
        return inputs.sliding_spec(B, dtype, H=H, Hkv=H, D=D, n_slots=S or 511)
    return inputs.full_spec(B, S, dtype, H=H, Hkv=H, D=D)


def oracle_step(x, write=False):
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    return oracle.layer_step(x.q, x.k, x.v, x.gate, kc, vc, x.pos, CODE[x.spec.dtype],
                             x.spec.kind == "sliding", x.spec.rot, x.spec.theta, write=write,
                             kv_scale=x.spec.kv_scale)


def gpu_unfused(x, kps=0, max_pos=None):
    """rope_apply -> decode_attn_* (pre-gate o) on device; returns (o, q_rot, k_rot)."""
    d = to_dev(x)
    ring = x.spec.kind == "sliding"
    desc = hswd.make_desc(d["k_cache"], keys_per_split=kps, kv_scale=d["kv_scale"])
    hswd.rope_apply(d["q"], d["k"], d["pos"], x.spec.rot, x.spec.theta)
    mp = int(x.pos.max()) if max_pos is None else max_pos
    ws = hswd.workspace(desc, ring, mp)
    if ring:
        o = hswd.decode_attn_sliding(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"],
                                     d["pos"], ws, desc=desc)
    else:
        o = hswd.decode_attn_full(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["pos"],
                                  mp, ws, desc=desc)
    assert hswd.check_errors(ws) == 0
    return o.cpu().numpy(), d["q"].cpu().numpy(), d["k"].cpu().numpy()


# ---------------------------------------------------------------------------
# the named small workloads
# ---------------------------------------------------------------------------
CASES = [
    # 1 stream, sliding, fp32 ring, position 600 (ring wrapped)
    ("sliding_1x600_f32", "sliding", 1, "f32", [600], None, 0),
    # 1 stream, full, fp16 cache, context 1024
    ("full_1x1024_f16", "full", 1, "f16", [1024], 1025, 0),
    # 64 streams, sliding, bf16, ragged positions in [1, 4096]
    ("sliding_64xragged_bf16", "sliding", 64, "bf16", "ragged", None, 0),
    # ragged full layer over several splits, with empty splits
    ("full_16xragged_bf16_kps128", "full", 16, "bf16", "ragged", 2049, 128),
    ("full_8xragged_f32_kps64", "full", 8, "f32", "ragged", 700, 64),
    ("sliding_8xragged_f16_kps128", "sliding", 8, "f16", "ragged", None, 128),
    ("full_4x_f16_d128", "full", 4, "f16", [5, 300, 1000, 77], 1001, 0),
    # fp8 e4m3 caches with per-head scales
    ("sliding_64xragged_fp8", "sliding", 64, "fp8", "ragged", None, 0),
    ("full_16xragged_fp8_kps128", "full", 16, "fp8", "ragged", 2049, 128),
    ("full_4x_fp8_d128", "full", 4, "fp8", [5, 300, 1000, 77], 1001, 0),
    # long chunks, ragged last chunk
    ("full_3x_bf16_kps4096", "full", 3, "bf16", [9000, 4097, 1], 9001, 4096),
    ("full_3x_fp8_kps8192", "full", 3, "fp8", [9000, 8192, 0], 9001, 8192),
]


@pytest.mark.parametrize("name,kind,B,dtype,pos,S,kps", CASES, ids=[c[0] for c in CASES])
def test_decode_attn_parity(name, kind, B, dtype, pos, S, kps):
    D = 128 if name.endswith("d128") else 256
    spec = spec_for(kind, B, dtype, S=S, D=D)
    if pos == "ragged":
        hi = 4096 if kind == "sliding" else spec.n_slots - 1
        pos = inputs.ragged_positions(B, 1, hi, seed=3)
        pos[0] = 1                                  # a nearly empty cache
    x = inputs.make_step(spec, pos, seed=zlib.crc32(name.encode()) % 1000)
    say("decode_attn %s pos=%s" % (name, list(x.pos[:8])))
    ref = oracle_step(x)
    o, q_rot, k_rot = gpu_unfused(x, kps=kps)
    assert_parity(o, ref["o_pre"], x, name)


def test_sliding_equals_full_on_same_history():
    """pos <= 511: a ring that never wrapped holds the same rows as an append
    cache; with one RoPE setting both kernels must agree."""
    B, S = 4, 511
    spec = inputs.sliding_spec(B, "bf16")
    x = inputs.make_step(spec, [1, 100, 300, 511], seed=7)
    ring_o, _, _ = gpu_unfused(x)
    y = inputs.make_step(spec, [1, 100, 300, 511], seed=7)
    y.spec = inputs.LayerSpec("full", B, 8, 8, 256, S + 1, "bf16", rot=256, theta=1e4)
    pad = np.full((B, 8, 1, 256), 0x7fc0, np.uint16)
    y.k_cache = np.concatenate([y.k_cache, pad], 2)
    y.v_cache = np.concatenate([y.v_cache, pad], 2)
    full_o, _, _ = gpu_unfused(y, max_pos=511)
    say("sliding vs full max diff %.3e" % np.max(np.abs(ring_o - full_o)))
    assert np.max(np.abs(ring_o - full_o)) < 1e-5


def test_wrapped_ring_equals_full_on_rolled_window():
    """pos >= 511: the ring's 511 slots, read in position order (slot
    (p - 511 + j) mod 511 for j = 0..510), as an append cache at pos 511,
    with the same rotated query, key and value: the ring kernel and the
    append kernel attend the same keys (a ring needs no reordering)."""
    B, S = 5, 511
    spec = inputs.sliding_spec(B, "bf16")
    pos = np.array([511, 600, 1000, 1021, 4096], np.int32)
    x = inputs.make_step(spec, pos, seed=8)
    d = to_dev(x)
    hswd.rope_apply(d["q"], d["k"], d["pos"], spec.rot, spec.theta)
    desc = hswd.make_desc(d["k_cache"])
    ws = hswd.workspace(desc, 1, 0)
    ring_o = hswd.decode_attn_sliding(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"],
                                      d["pos"], ws, desc=desc).cpu().numpy()
    order = (pos[:, None] - S + np.arange(S)[None, :]) % S          # [B, 511] slots
    pad = np.full((B, 8, 1, 256), 0x7fc0, np.uint16)
    kr = np.stack([x.k_cache[b][:, order[b]] for b in range(B)])
    vr = np.stack([x.v_cache[b][:, order[b]] for b in range(B)])
    kf = cache_to_dev(np.concatenate([kr, pad], 2), "bf16")
    vf = cache_to_dev(np.concatenate([vr, pad], 2), "bf16")
    fdesc = hswd.make_desc(kf)
    fws = hswd.workspace(fdesc, 0, S)
    fpos = torch.full((B,), S, dtype=torch.int32, device="cuda")
    full_o = hswd.decode_attn_full(d["q"], d["k"], d["v"], kf, vf, fpos, S, fws,
                                   desc=fdesc).cpu().numpy()
    assert hswd.check_errors(ws) == 0 and hswd.check_errors(fws) == 0
    say("wrapped ring vs rolled full max diff %.3e" % np.max(np.abs(ring_o - full_o)))
    assert np.max(np.abs(ring_o - full_o)) < 1e-5


def test_single_key_returns_rounded_value():
    """pos 0: nothing cached; the output is the new entry's value, bit for bit."""
    for kind, dtype in [("sliding", "bf16"), ("full", "f16"), ("sliding", "f32")]:
        spec = spec_for(kind, 3, dtype, S=8 if kind == "full" else None)
        x = inputs.make_step(spec, [0, 0, 0], seed=9)
        say("single key %s %s" % (kind, dtype))
        o, _, _ = gpu_unfused(x, max_pos=0)
        vh = oracle.decode(CODE[dtype], oracle.round_to(CODE[dtype], x.v))
        assert np.array_equal(o.astype(np.float64), vh)


def test_zero_query_gives_mean():
    """q = 0: all scores equal; the output is the mean of the attended values."""
    spec = inputs.sliding_spec(4, "bf16")
    x = inputs.make_step(spec, [3, 511, 700, 100], seed=10)
    x.q[:] = 0
    say("zero query")
    o, _, _ = gpu_unfused(x)
    ref = oracle_step(x)["o_pre"]
    assert_parity(o, ref, x, "zero query")


def test_partials_and_merge_match_oracle_split_form():
    """Split partials of the cached keys (a5) and their merge (a7)."""
    B, S, kps = 4, 1300, 256
    spec = inputs.full_spec(B, S, "bf16")
    x = inputs.make_step(spec, [1299, 5, 700, 256], seed=11)
    d = to_dev(x)
    hswd.rope_apply(d["q"], d["k"], d["pos"], spec.rot, spec.theta)
    desc = hswd.make_desc(d["k_cache"], keys_per_split=kps)
    say("partials B=%d kps=%d" % (B, kps))
    po, pml = hswd.decode_attn_partials(d["q"], d["k_cache"], d["v_cache"], d["pos"], 0,
                                        max_pos=1299, desc=desc)
    po, pml = po.cpu().numpy(), pml.cpu().numpy()
    n = po.shape[2]
    assert n == math.ceil(1299 / kps)
    q_rot = d["q"].cpu().numpy().astype(np.float64)
    for b in range(B):
        p = int(x.pos[b])
        for h in range(spec.H):
            for c in range(n):
                j0, j1 = c * kps, min((c + 1) * kps, p)
                m, l, o = oracle.partial(q_rot[b, h], x.k_cache[b, h], x.v_cache[b, h],
                                         CODE["bf16"], j0, j1, 1 / 16)
                if j1 <= j0:
                    assert pml[b, h, c, 0] == -np.inf and pml[b, h, c, 1] == 0
                    assert np.all(po[b, h, c] == 0)
                    continue
                assert abs(pml[b, h, c, 0] - m) < 1e-5 * (1 + abs(m))
                # o and l are relative to each side's own max; rescale to compare
                scale = math.exp(pml[b, h, c, 0] - m)
                assert abs(pml[b, h, c, 1] * scale - l) < 1e-5 * l
                assert np.max(np.abs(po[b, h, c] * scale - o)) < 1e-5 * np.max(np.abs(o))
    merged = hswd.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pml).cuda())
    merged = merged.cpu().numpy()
    for b in range(B):
        if int(x.pos[b]) == 0:
            continue
        for h in range(spec.H):
            ref = oracle.merge(pml[b, h, :, 0].astype(np.float64), pml[b, h, :, 1], po[b, h])
            assert np.max(np.abs(merged[b, h] - ref)) < 1e-5 * np.max(np.abs(ref))


@pytest.mark.parametrize("kind,dtype,pos,S,kps", [
    ("sliding", "bf16", "ragged", None, 0),
    ("sliding", "f32", [600, 3], None, 128),
    ("full", "bf16", "ragged", 3000, 0),
    ("full", "f16", [1024, 1, 0, 2999], 3000, 256),
    ("sliding", "fp8", "ragged", None, 0),
    ("full", "fp8", [1024, 1, 0, 2999], 3000, 256),
])
def test_layer_step_fused_matches_oracle_and_unfused(kind, dtype, pos, S, kps):
    """The one-launch layer step: gated output against the oracle, the stored
    entry bit for bit, and the same bits as the four separate entries."""
    B = 12 if pos == "ragged" else len(pos)
    spec = spec_for(kind, B, dtype, S=S)
    if pos == "ragged":
        pos = inputs.ragged_positions(B, 0, 4096 if kind == "sliding" else S - 1, seed=12)
    x = inputs.make_step(spec, pos, seed=13)
    ring = kind == "sliding"
    ref = oracle_step(x, write=True)
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"], keys_per_split=kps, kv_scale=d["kv_scale"])
    mp = int(x.pos.max())
    ws = hswd.workspace(desc, ring, mp)
    say("layer_step fused %s %s pos=%s" % (kind, dtype, list(x.pos[:6])))
    out = hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                          d["pos"], ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
    assert hswd.check_errors(ws) == 0
    out = out.cpu().numpy()
    assert_parity(out, ref["out"], x, "fused step")
    kc, vc = cache_to_host(d["k_cache"]), cache_to_host(d["v_cache"])

    # unfused sequence on fresh copies: rope -> attend -> gate -> write
    e = to_dev(x)
    hswd.rope_apply(e["q"], e["k"], e["pos"], spec.rot, spec.theta)
    ws2 = hswd.workspace(desc, ring, mp)
    if ring:
        o = hswd.decode_attn_sliding(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"],
                                     e["pos"], ws2, desc=desc)
    else:
        o = hswd.decode_attn_full(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"], e["pos"],
                                  mp, ws2, desc=desc)
    g = hswd.head_gate(o, e["gate"])
    hswd.kv_slot_write(e["k_cache"], e["v_cache"], e["k"], e["v"], e["pos"], ring, ws2,
                       desc=desc)
    assert hswd.check_errors(ws2) == 0
    assert np.array_equal(g.cpu().numpy(), out), "fused and unfused outputs differ"
    kc2, vc2 = cache_to_host(e["k_cache"]), cache_to_host(e["v_cache"])
    assert np.array_equal(kc.view(np.uint8), kc2.view(np.uint8))

    # the stored entry equals the oracle's rounding of the GPU's rotated key
    k_rot = e["k"].cpu().numpy()
    for b in range(B):
        p = int(x.pos[b])
        row = p % spec.n_slots if ring else p
        sc = spec.kv_scale
        want_k = entry_codes(k_rot[b], dtype, None if sc is None else sc[0][:, None])
        want_v = entry_codes(x.v[b], dtype, None if sc is None else sc[1][:, None])
        if dtype == "f32":
            assert np.array_equal(kc[b, :, row].view(np.uint32), want_k.view(np.uint32))
            assert np.array_equal(vc[b, :, row].view(np.uint32), want_v.view(np.uint32))
        else:
            assert np.array_equal(kc[b, :, row], want_k)
            assert np.array_equal(vc[b, :, row], want_v)
        # every other row is untouched
        others = np.ones(spec.n_slots, bool)
        others[row] = False
        kb = kc[b][:, others].view(np.uint8)
        xb = x.k_cache[b][:, others].view(np.uint8)
        assert np.array_equal(kb, xb)


@pytest.mark.parametrize("kind,dtype", [("sliding", "f32"), ("sliding", "bf16"),
                                        ("full", "f16"), ("sliding", "fp8")])
def test_multistep_against_brute_force(kind, dtype):
    """Several steps through the ring's wrap, driven on the GPU with the fused
    layer step (read, then write), against the brute force over the raw
    history: a 4-token window (3 slots), D = 256."""
    rng = np.random.default_rng(50)
    H, D, steps, W = 2, 256, 12, 4
    ring = kind == "sliding"
    S = W - 1 if ring else steps
    rot, theta = (D, 1e4) if ring else (D // 4, 5e6)
    hist = [(rng.standard_normal((H, D)).astype(np.float32),
             rng.standard_normal((H, D)).astype(np.float32),
             rng.standard_normal((H, D)).astype(np.float32)) for _ in range(steps)]
    gate = rng.standard_normal(H).astype(np.float32)
    hist_py = [(q.tolist(), k.tolist(), v.tolist()) for q, k, v in hist]
    sd = oracle.storage_dtype(CODE[dtype])
    nan = inputs.nan_bits(dtype)
    kc = cache_to_dev(np.full((1, H, S, D), nan, sd), dtype)
    vc = cache_to_dev(np.full((1, H, S, D), nan, sd), dtype)
    ksc = inputs.default_fp8_scales(H) if dtype == "fp8" else None
    ksc_dev = None if ksc is None else f32_dev(ksc)
    desc = hswd.make_desc(kc, kv_scale=ksc_dev)
    ws = hswd.workspace(desc, ring, S - 1)
    say("multistep %s %s" % (kind, dtype))
    for p in range(steps):
        q, k, v = hist[p]
        out = hswd.layer_step(f32_dev(q[None]), f32_dev(k[None]), f32_dev(v[None]),
                              f32_dev(gate[None]), kc, vc, i32_dev([p]), ring, rot, theta, ws,
                              max_pos=0 if ring else S - 1, desc=desc)
        ref = np.array(brute.step(hist_py, p, W if ring else None, H, H, rot, theta, dtype,
                                  1 / 16, gate.tolist(), None if ksc is None else ksc.tolist()))
        got = out.cpu().numpy()[0]
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        assert err < (1e-5 if dtype == "f32" else 2e-3 / 4), (p, err)
    assert hswd.check_errors(ws) == 0


def test_deterministic_and_batch_invariant():
    """Same inputs twice: same bits.  A stream alone and inside a batch of
    64: same bits (the split count never depends on the batch)."""
    spec = inputs.full_spec(64, 2100, "bf16")
    pos = inputs.ragged_positions(64, 1, 2099, seed=14)
    x = inputs.make_step(spec, pos, seed=15)
    say("determinism")
    a, _, _ = gpu_unfused(x, max_pos=2099)
    b, _, _ = gpu_unfused(x, max_pos=2099)
    assert np.array_equal(a, b)
    for s in (0, 17, 63):
        one = inputs.StepInputs(inputs.full_spec(1, 2100, "bf16"), x.pos[s:s + 1], x.q[s:s + 1],
                                x.k[s:s + 1], x.v[s:s + 1], x.gate[s:s + 1],
                                x.k_cache[s:s + 1], x.v_cache[s:s + 1])
        solo, _, _ = gpu_unfused(one, max_pos=2099)
        assert np.array_equal(solo[0], a[s]), s


def test_max_pos_flag():
    """A device position above the host bound is reported, not silently used."""
    spec = inputs.full_spec(2, 2000, "bf16")
    x = inputs.make_step(spec, [100, 1500], seed=16)
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"])
    ws = hswd.workspace(desc, 0, 600)
    say("max_pos flag")
    hswd.decode_attn_full(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["pos"], 600, ws,
                          desc=desc)
    assert hswd.check_errors(ws) & hswd.binding.FLAG_MAX_POS


@pytest.mark.parametrize("kind,dtype,S,kps", [("full", "bf16", 3000, 256),
                                              ("sliding", "f32", None, 128),
                                              ("full", "f16", 2100, 0)])
def test_work_split_never_changes_bits(kind, dtype, S, kps):
    """Chunks per workgroup only moves work between workgroups: one
    workgroup per chunk, several chunks each, or the whole range in one must
    give the same bits, in both the attention entry and the fused step."""
    B = 6
    spec = spec_for(kind, B, dtype, S=S)
    hi = 4096 if kind == "sliding" else S - 1
    pos = inputs.ragged_positions(B, 0, hi, seed=17)
    x = inputs.make_step(spec, pos, seed=18)
    ring = kind == "sliding"
    mp = int(x.pos.max())
    outs, steps, caches = [], [], []
    for cpw in (1, 2, 5, 64, 0):
        d = to_dev(x)
        desc = hswd.make_desc(d["k_cache"], keys_per_split=kps, chunks_per_workgroup=cpw)
        say("work split %s %s cpw=%d" % (kind, dtype, cpw))
        ws = hswd.workspace(desc, ring, mp)
        out = hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                              d["pos"], ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
        steps.append(out.cpu().numpy())
        caches.append(cache_to_host(d["k_cache"]))
        e = to_dev(x)
        hswd.rope_apply(e["q"], e["k"], e["pos"], spec.rot, spec.theta)
        if ring:
            o = hswd.decode_attn_sliding(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"],
                                         e["pos"], ws, desc=desc)
        else:
            o = hswd.decode_attn_full(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"],
                                      e["pos"], mp, ws, desc=desc)
        assert hswd.check_errors(ws) == 0
        outs.append(o.cpu().numpy())
    for i in range(1, len(outs)):
        assert np.array_equal(outs[0], outs[i]), i
        assert np.array_equal(steps[0], steps[i]), i
        assert np.array_equal(caches[0].view(np.uint8), caches[i].view(np.uint8)), i
    ref = oracle_step(x)
    assert_parity(outs[0], ref["o_pre"], x, "work split")


@pytest.mark.parametrize("kind,dtype", [("sliding", "bf16"), ("full", "fp8")])
def test_bound_layer_step_matches_plain_call(kind, dtype):
    """bind_layer_step marshals once and launches the same entry point: the
    output and the written entry equal those of layer_step bit for bit, on
    each of two launches."""
    B = 5
    spec = spec_for(kind, B, dtype, S=1500)
    hi = 3000 if kind == "sliding" else 1499
    x = inputs.make_step(spec, inputs.ragged_positions(B, 1, hi, seed=19), seed=20)
    ring = kind == "sliding"
    mp = int(x.pos.max())
    d1, d2 = to_dev(x), to_dev(x)
    desc1 = hswd.make_desc(d1["k_cache"], kv_scale=d1["kv_scale"])
    desc2 = hswd.make_desc(d2["k_cache"], kv_scale=d2["kv_scale"])
    ws1, ws2 = hswd.workspace(desc1, ring, mp), hswd.workspace(desc2, ring, mp)
    say("bound layer step %s %s" % (kind, dtype))
    call = hswd.bind_layer_step(d2["q"], d2["k"], d2["v"], d2["gate"], d2["k_cache"],
                                d2["v_cache"], d2["pos"], ring, spec.rot, spec.theta, ws2,
                                max_pos=mp, desc=desc2)
    # two launches each; in a ring past its capacity the first overwrites an
    # attended slot, so both sides advance together
    for _ in range(2):
        ref = hswd.layer_step(d1["q"], d1["k"], d1["v"], d1["gate"], d1["k_cache"],
                              d1["v_cache"], d1["pos"], ring, spec.rot, spec.theta, ws1,
                              max_pos=mp, desc=desc1)
        got = call()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
        assert np.array_equal(cache_to_host(d2["k_cache"]), cache_to_host(d1["k_cache"]))
        assert np.array_equal(cache_to_host(d2["v_cache"]), cache_to_host(d1["v_cache"]))
    assert hswd.check_errors(ws2) == 0


@pytest.mark.parametrize("kind,B,dtype,pos,S,D", [
    ("sliding", 1, "f32", [600], None, 256),            # one stream, f32 ring
    ("full", 1, "f16", [1024], 1025, 256),              # one stream, f16 full layer
    ("sliding", 8, "bf16", [131072] * 8, None, 256),    # 8 rings past capacity
    ("full", 3, "fp8", [1099, 3, 600], 1100, 256),      # fp8, few keys, empty chunks
    ("full", 2, "bf16", [700, 2], 1025, 128),           # D = 128, a stream with 2 keys
    ("full", 1, "bf16", [1280], 1281, 128),             # 3 chunks: an odd count
])
def test_small_batch_work_split_never_changes_bits(kind, B, dtype, pos, S, D):
    """The single-stream and few-stream shapes, where the library spreads a
    (stream, kv head) over several workgroups and merges their chunk
    partials: the library's split, one workgroup per chunk, and one
    workgroup streaming every chunk give the same bits, in the fused step
    (with the gate given, and with the gate projected in the launch) and in
    the attention entry; and match the oracle."""
    spec = spec_for(kind, B, dtype, S=S, D=D)
    x = inputs.make_step(spec, pos, seed=23)
    ring = kind == "sliding"
    mp = int(x.pos.max())
    gx, gw = inputs.gate_inputs(B, 2048, spec.H, seed=24)
    results = []
    for cpw in (0, 1, 64):
        d = to_dev(x)
        desc = hswd.make_desc(d["k_cache"], chunks_per_workgroup=cpw, kv_scale=d["kv_scale"])
        n = hswd.num_splits(desc, ring, mp)
        say("small-batch split %s %s B=%d D=%d pos=%s: %d chunks, cpw=%d" % (
            kind, dtype, B, D, list(x.pos), n, cpw))
        ws = hswd.workspace(desc, ring, mp)
        out = hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                              d["pos"], ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
        e = to_dev(x)
        out_g = hswd.layer_step_gproj(e["q"], e["k"], e["v"], f32_dev(gx), f32_dev(gw),
                                      e["k_cache"], e["v_cache"], e["pos"], ring, spec.rot,
                                      spec.theta, ws, max_pos=mp, desc=desc)
        f = to_dev(x)
        hswd.rope_apply(f["q"], f["k"], f["pos"], spec.rot, spec.theta)
        if ring:
            o = hswd.decode_attn_sliding(f["q"], f["k"], f["v"], f["k_cache"], f["v_cache"],
                                         f["pos"], ws, desc=desc)
        else:
            o = hswd.decode_attn_full(f["q"], f["k"], f["v"], f["k_cache"], f["v_cache"],
                                      f["pos"], mp, ws, desc=desc)
        assert hswd.check_errors(ws) == 0
        results.append([out.cpu().numpy(), out_g.cpu().numpy(), o.cpu().numpy(),
                        cache_to_host(d["k_cache"]), cache_to_host(d["v_cache"])])
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    ref = oracle_step(x)
    assert_parity(results[0][2], ref["o_pre"], x, "small-batch split, attention entry")
    assert_parity(results[0][0], ref["out"], x, "small-batch split, fused step")


@pytest.mark.parametrize("dtype,H", [("bf16", 8), ("fp8", 32)])
def test_packed_split_never_changes_bits(dtype, H):
    """Long append caches under the default chunking (a launch bound of
    32768 keys or more) take the packed split, whose deal gives the streams
    different workgroup counts from their positions: its bits equal those
    of one workgroup per chunk and of 64 chunks per workgroup (fixed splits
    sized for the longest stream), in the fused step and the attention
    entry, with the written entries; every head matches the oracle (8 kv
    heads; 32 query heads: the 4-head kernel)."""
    B, S = 12, 50001
    spec = inputs.full_spec(B, S, dtype, H=H, Hkv=8, D=128)
    pos = inputs.ragged_positions(B, 0, S - 1, seed=26)
    pos[:3] = [S - 1, 0, 3]                  # the capacity, empty, a few keys
    x = inputs.make_step(spec, pos, seed=27)
    mp = int(x.pos.max())
    results = []
    for cpw in (0, 1, 64):
        d = to_dev(x)
        desc = hswd.make_desc(d["k_cache"], n_heads=H, chunks_per_workgroup=cpw,
                              kv_scale=d["kv_scale"])
        say("packed split %s H=%d B=%d pos=%s..., cpw=%d" % (dtype, H, B, list(x.pos[:5]), cpw))
        ws = hswd.workspace(desc, 0, mp)
        out = hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                              d["pos"], 0, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
        f = to_dev(x)
        hswd.rope_apply(f["q"], f["k"], f["pos"], spec.rot, spec.theta)
        o = hswd.decode_attn_full(f["q"], f["k"], f["v"], f["k_cache"], f["v_cache"], f["pos"],
                                  mp, ws, desc=desc)
        assert hswd.check_errors(ws) == 0
        results.append([out.cpu().numpy(), o.cpu().numpy(), cache_to_host(d["k_cache"]),
                        cache_to_host(d["v_cache"])])
        del d, f
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    ref = oracle_step(x)
    assert_parity(results[0][1], ref["o_pre"], x, "packed split, attention entry")
    assert_parity(results[0][0], ref["out"], x, "packed split, fused step")


def _stream_chunk(n, floor=256):
    """The header's default chunk of an append-cache stream with n valid keys
    (bf16, D = 256, 8 kv heads, one query head per each: floor of four 64-key
    quanta): the smallest power of two >= max(floor, ceil(n / 32)), at most
    1024 below 131072 keys, 2048 below 524288 and 8192 from there."""
    cap = 1024 if n < 131072 else (2048 if n < 524288 else 8192)
    k = floor
    while k < -(-n // 32) and k < cap:
        k *= 2
    return k


def test_very_long_streams_take_longer_chunks():
    """Streams of 2^19 keys or more take 8192-key chunks (fewer partials for
    the last workgroup to fold), the stream one key below them 2048-key
    chunks: in one batch with shorter streams each stream gives the bits it
    gives decoded alone and under a fixed split (one workgroup per chunk),
    and every head matches the oracle (bf16, 128 dims)."""
    S = (1 << 19) + 1
    pos = np.array([1 << 19, (1 << 19) - 1, 70000, 0], np.int32)
    spec = inputs.full_spec(len(pos), S, "bf16", D=128)
    t = inputs.device_step(spec, pos, seed=28, device="cuda")
    kc_host, vc_host = cache_to_host(t["k_cache"]), cache_to_host(t["v_cache"])
    q, k, v, gate = (t[n].cpu().numpy() for n in ("q", "k", "v", "gate"))
    mp = int(pos.max())
    q_rot, k_rot = t["q"].clone(), t["k"].clone()
    hswd.rope_apply(q_rot, k_rot, t["pos"], spec.rot, spec.theta)
    outs = []
    for cpw in (0, 1):
        desc = hswd.make_desc(t["k_cache"], chunks_per_workgroup=cpw)
        say("very long streams: pos %s, %d chunks, cpw=%d" % (list(pos), hswd.num_splits(desc, 0, mp),
                                                              cpw))
        ws = hswd.workspace(desc, 0, mp)
        outs.append(hswd.decode_attn_full(q_rot, k_rot, t["v"], t["k_cache"], t["v_cache"],
                                          t["pos"], mp, ws, desc=desc).cpu().numpy())
        assert hswd.check_errors(ws) == 0
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8))
    for b, p in enumerate(pos):
        sl = slice(b, b + 1)
        d1 = hswd.make_desc(t["k_cache"][sl])
        ws1 = hswd.workspace(d1, 0, max(int(p), 1))
        o1 = hswd.decode_attn_full(q_rot[sl].contiguous(), k_rot[sl].contiguous(),
                                   t["v"][sl].contiguous(), t["k_cache"][sl], t["v_cache"][sl],
                                   t["pos"][sl].contiguous(), max(int(p), 1), ws1, desc=d1)
        assert np.array_equal(o1.cpu().numpy()[0], outs[0][b]), b
    r = oracle.layer_step(q, k, v, gate, kc_host, vc_host, pos, CODE["bf16"], 0, spec.rot,
                          spec.theta, write=False)
    x = inputs.StepInputs(spec, pos, q, k, v, gate, kc_host, vc_host)
    assert_parity(outs[0], r["o_pre"], x, "very long streams")


def test_stream_chunks_follow_their_own_positions():
    """Append caches under the default chunking cut each stream's keys into
    chunks sized from its own position (about 32 of them): a stream far below
    the cache's capacity still spreads over many workgroups.  A stream decoded
    alone (its own position as the launch's bound) gives the same bits as in
    a batch whose longest stream is at the capacity; every head matches the
    oracle; the partials entry's chunks follow each stream's own size."""
    S = 131073
    pos = np.array([5000, 131072, 37, 70000], np.int32)
    spec = inputs.full_spec(len(pos), S, "bf16")
    t = inputs.device_step(spec, pos, seed=25, device="cuda")
    kc_host, vc_host = cache_to_host(t["k_cache"]), cache_to_host(t["v_cache"])
    q, k, v, gate = (t[n].cpu().numpy() for n in ("q", "k", "v", "gate"))
    mp = int(pos.max())
    desc = hswd.make_desc(t["k_cache"])
    n_grid = hswd.num_splits(desc, 0, mp)
    say("per-stream chunks: pos %s, launch sized for %d chunks" % (list(pos), n_grid))
    ws = hswd.workspace(desc, 0, mp)
    q_rot = t["q"].clone()
    k_rot = t["k"].clone()
    hswd.rope_apply(q_rot, k_rot, t["pos"], spec.rot, spec.theta)
    o_batch = hswd.decode_attn_full(q_rot, k_rot, t["v"], t["k_cache"], t["v_cache"], t["pos"],
                                    mp, ws, desc=desc).cpu().numpy()
    po, pml = hswd.decode_attn_partials(q_rot, t["k_cache"], t["v_cache"], t["pos"], 0,
                                        max_pos=mp, desc=desc)
    assert hswd.check_errors(ws) == 0
    po, pml = po.cpu().numpy(), pml.cpu().numpy()
    assert po.shape[2] == n_grid
    # each stream alone, its own position the launch's bound
    for b, p in enumerate(pos):
        sl = slice(b, b + 1)
        d1 = hswd.make_desc(t["k_cache"][sl])
        ws1 = hswd.workspace(d1, 0, int(p))
        o1 = hswd.decode_attn_full(q_rot[sl].contiguous(), k_rot[sl].contiguous(),
                                   t["v"][sl].contiguous(), t["k_cache"][sl], t["v_cache"][sl],
                                   t["pos"][sl].contiguous(), int(p), ws1, desc=d1)
        assert np.array_equal(o1.cpu().numpy()[0], o_batch[b]), b
    # every head against the oracle
    r = oracle.layer_step(q, k, v, gate, kc_host, vc_host, pos, CODE["bf16"], 0, spec.rot,
                          spec.theta, write=False)
    x = inputs.StepInputs(spec, pos, q, k, v, gate, kc_host, vc_host)
    assert_parity(o_batch, r["o_pre"], x, "per-stream chunks")
    # the partials' chunks: each stream's own size, empty past its keys
    qr = q_rot.cpu().numpy().astype(np.float64)
    for b, p in enumerate(pos):
        K = _stream_chunk(int(p))
        nb = -(-int(p) // K)
        for h in (0, spec.H - 1):
            for c in range(n_grid):
                if c >= nb:
                    assert pml[b, h, c, 0] == -np.inf and pml[b, h, c, 1] == 0, (b, c)
                    assert np.all(po[b, h, c] == 0)
                    continue
                m, l, o = oracle.partial(qr[b, h], kc_host[b, h], vc_host[b, h], CODE["bf16"],
                                         c * K, min((c + 1) * K, int(p)), 1 / 16)
                assert abs(pml[b, h, c, 0] - m) < 1e-5 * (1 + abs(m)), (b, h, c)
                sc = math.exp(pml[b, h, c, 0] - m)
                assert abs(pml[b, h, c, 1] * sc - l) < 1e-5 * l, (b, h, c)
                assert np.max(np.abs(po[b, h, c] * sc - o)) < 1e-5 * np.max(np.abs(o)), (b, h, c)
