"""GPU parity of grouped-query attention (H / Hkv query heads per kv head,
the talker commit's query reshape; groups 2 and 4 and larger ones): the fused layer step and the
separate entries against the oracle (which maps query head h to kv head
h // G), the stored entry bit for bit, the cross-workgroup merge, and the
property that a group reads the same result as its kv head repeated."""
import numpy as np
import pytest

import hybrid_sliding_window_decode_amd as hswd
import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import (CODE, assert_parity, cache_to_host, entry_codes, f32_dev, i32_dev,
                      say, to_dev)

pytestmark = pytest.mark.gpu


def gqa_spec(kind, B, dtype, G, D=256, S=None, H=8):
    if kind == "sliding":
        return inputs.sliding_spec(B, dtype, H=H, Hkv=H // G, D=D)
    return inputs.full_spec(B, S, dtype, H=H, Hkv=H // G, D=D)


def oracle_step(x, write=False):
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    return oracle.layer_step(x.q, x.k, x.v, x.gate, kc, vc, x.pos, CODE[x.spec.dtype],
                             x.spec.kind == "sliding", x.spec.rot, x.spec.theta, write=write,
                             kv_scale=x.spec.kv_scale)


def positions(kind, B, S, pos, seed):
    if pos == "ragged":
        hi = 4096 if kind == "sliding" else S - 1
        return inputs.ragged_positions(B, 0, hi, seed=seed)
    return pos


@pytest.mark.parametrize("kind,dtype,G,D,B,pos,S,kps", [
    ("sliding", "bf16", 4, 256, 12, "ragged", None, 0),
    ("sliding", "f16", 2, 128, 9, "ragged", None, 0),
    ("full", "bf16", 2, 256, 10, "ragged", 3000, 0),
    ("full", "f16", 4, 128, 4, [1024, 1, 0, 2999], 3000, 256),
    # two streams, long context: several workgroups per (stream, kv head),
    # merged by the last to arrive
    ("full", "bf16", 4, 256, 2, [19999, 7001], 20000, 0),
    # fp8 e4m3 caches with per-head scales (8-byte lane chunks)
    ("sliding", "fp8", 4, 256, 12, "ragged", None, 0),
    ("full", "fp8", 2, 128, 6, "ragged", 3000, 256),
    ("full", "fp8", 4, 256, 2, [19999, 9000], 20000, 0),
    # bf16 at D = 128: the 4-head kernel's value product on the matrix cores
    # with each probability split into two bf16 parts
    ("full", "bf16", 4, 128, 3, [4000, 17, 2048], 4001, 0),
    ("sliding", "bf16", 4, 128, 5, "ragged", None, 0),
    # fp8, 2 heads per kv head: the 4-head matrix-core kernel with two heads
    # idle, over rings and append caches
    ("sliding", "fp8", 2, 256, 6, "ragged", None, 0),
    ("full", "fp8", 2, 256, 3, [4000, 17, 2048], 4001, 0),
    # fp8 at D = 128: 64-key tiles, two 32-key value products per tile
    ("full", "fp8", 4, 128, 3, [4000, 17, 2048], 4001, 0),
    ("sliding", "fp8", 4, 128, 5, "ragged", None, 0),
])
def test_gqa_layer_step(kind, dtype, G, D, B, pos, S, kps):
    check_layer_step(kind, dtype, G, D, B, pos, S, kps)


# Groups without a kernel of their own: 3 runs the 4-head kernel with one
# head idle, 5 to 7 the 8-head kernel with heads idle; 16 runs the 8-head
# kernel in two pieces (one workgroup each, the last to finish writes the
# entry); with cross-workgroup merges, 128 and 256 dims, every cache type.
@pytest.mark.parametrize("kind,dtype,G,D,B,pos,S,kps,H", [
    ("sliding", "bf16", 3, 256, 6, "ragged", None, 0, 12),
    ("full", "f16", 3, 128, 3, [1024, 1, 2999], 3000, 256, 24),
    ("full", "bf16", 8, 256, 5, "ragged", 3000, 0, 32),
    ("sliding", "fp8", 8, 256, 6, "ragged", None, 0, 16),
    ("full", "fp8", 6, 256, 3, [2999, 0, 1500], 3000, 0, 24),
    ("full", "bf16", 5, 256, 2, [19999, 7001], 20000, 0, 10),
    ("sliding", "f16", 16, 128, 4, "ragged", None, 0, 32),
    ("full", "fp8", 8, 256, 2, [19999, 7001], 20000, 0, 16),
    ("full", "fp8", 8, 128, 4, "ragged", 3000, 0, 64),
    ("sliding", "fp8", 16, 256, 4, "ragged", None, 0, 32),
    ("full", "fp8", 5, 256, 3, [2999, 1, 1500], 3000, 0, 10),
    # the 8-head kernel over 16-bit caches: 128 dims (two V tiles in
    # flight), 256 dims (one), merges across workgroups, pieces of 16
    ("full", "f16", 8, 128, 3, [4000, 17, 2048], 4001, 0, 64),
    ("sliding", "bf16", 7, 128, 5, "ragged", None, 0, 56),
    ("full", "bf16", 8, 256, 2, [19999, 7001], 20000, 0, 64),
    ("full", "f16", 16, 256, 2, [6000, 4097], 6001, 0, 32),
    ("sliding", "bf16", 16, 256, 3, "ragged", None, 0, 64),
    # long chunks, ragged last chunk: the 4- and 8-head kernels
    ("full", "bf16", 4, 256, 2, [9000, 4097], 9001, 4096, 32),
    ("full", "fp8", 8, 256, 2, [9000, 2049], 9001, 4096, 64),
    ("full", "bf16", 8, 256, 2, [9000, 2049], 9001, 4096, 64),
])
def test_gqa_large_groups(kind, dtype, G, D, B, pos, S, kps, H):
    check_layer_step(kind, dtype, G, D, B, pos, S, kps, H=H)


# Sharply peaked attention: the query scaled by 20 makes the scores ~N(0, 400),
# so each head's softmax is nearly one-hot and most weights underflow; the
# running max moves by large steps.  One head per kv head and grouped.
@pytest.mark.parametrize("kind,dtype,G,D,B,pos,S,kps", [
    ("sliding", "bf16", 1, 256, 8, "ragged", None, 0),
    ("full", "bf16", 1, 256, 6, "ragged", 3000, 0),
    ("full", "fp8", 1, 256, 6, "ragged", 3000, 0),
    ("full", "bf16", 1, 256, 2, [19999, 7001], 20000, 0),
    ("sliding", "fp8", 4, 256, 8, "ragged", None, 0),
    ("full", "bf16", 4, 256, 4, "ragged", 3000, 0),
    ("full", "bf16", 8, 256, 3, "ragged", 3000, 0),
    ("sliding", "fp8", 8, 256, 4, "ragged", None, 0),
    ("full", "fp8", 4, 128, 3, "ragged", 3000, 0),
    ("full", "fp8", 8, 128, 3, "ragged", 3000, 0),
    ("full", "f16", 2, 128, 4, "ragged", 3000, 256),
    ("full", "bf16", 4, 128, 3, "ragged", 3000, 0),
    ("full", "f16", 4, 128, 3, "ragged", 3000, 0),
])
def test_sharp_softmax(kind, dtype, G, D, B, pos, S, kps):
    check_layer_step(kind, dtype, G, D, B, pos, S, kps, q_mult=20.0)


def check_layer_step(kind, dtype, G, D, B, pos, S, kps, H=8, q_mult=1.0):
    """Fused step vs oracle; the same bits as rope -> attend -> gate -> write;
    the stored entry equals the oracle's rounding of the rotated key."""
    spec = gqa_spec(kind, B, dtype, G, D=D, S=S, H=H)
    x = inputs.make_step(spec, positions(kind, B, S, pos, 21), seed=22 + G)
    x.q *= np.float32(q_mult)
    ring = kind == "sliding"
    mp = int(x.pos.max())
    ref = oracle_step(x, write=True)
    d = to_dev(x)
    desc = hswd.make_desc(d["k_cache"], n_heads=spec.H, keys_per_split=kps,
                          kv_scale=d["kv_scale"])
    ws = hswd.workspace(desc, ring, mp)
    say("gqa layer_step %s %s G=%d D=%d B=%d pos=%s" % (kind, dtype, G, D, B, list(x.pos[:6])))
    out = hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                          d["pos"], ring, spec.rot, spec.theta, ws, max_pos=mp, desc=desc)
    assert hswd.check_errors(ws) == 0
    out = out.cpu().numpy()
    assert_parity(out, ref["out"], x, "gqa fused step")

    e = to_dev(x)
    hswd.rope_apply(e["q"], e["k"], e["pos"], spec.rot, spec.theta)
    ws2 = hswd.workspace(desc, ring, mp)
    if ring:
        o = hswd.decode_attn_sliding(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"],
                                     e["pos"], ws2, desc=desc)
    else:
        o = hswd.decode_attn_full(e["q"], e["k"], e["v"], e["k_cache"], e["v_cache"], e["pos"],
                                  mp, ws2, desc=desc)
    assert_parity(o.cpu().numpy(), ref["o_pre"], x, "gqa attention entry")
    g = hswd.head_gate(o, e["gate"])
    hswd.kv_slot_write(e["k_cache"], e["v_cache"], e["k"], e["v"], e["pos"], ring, ws2,
                       desc=desc)
    assert hswd.check_errors(ws2) == 0
    assert np.array_equal(g.cpu().numpy(), out), "fused and unfused outputs differ"
    kc = cache_to_host(d["k_cache"])
    # bit patterns (an f32 cache's unwritten rows hold NaN)
    same = lambda a, b: np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                       np.ascontiguousarray(b).view(np.uint8))
    assert same(kc, cache_to_host(e["k_cache"]))
    assert same(cache_to_host(d["v_cache"]), cache_to_host(e["v_cache"]))
    k_rot = e["k"].cpu().numpy()
    ksc = None if spec.kv_scale is None else spec.kv_scale[0][:, None]
    for b in range(B):
        p = int(x.pos[b])
        row = p % spec.n_slots if ring else p
        assert np.array_equal(kc[b, :, row], entry_codes(k_rot[b], dtype, ksc))


# A group split into pieces (one workgroup per piece in one launch; the
# last piece to finish writes the entry): consecutive steps on one
# workspace, each against the oracle stepping the same history, so the
# arrival counters must be back at zero after every call and each entry
# must land before the next step reads it.  Sliding rings are full (the
# overwritten slot is still in the window when it is read).
@pytest.mark.parametrize("kind,dtype,G,D,B,pos,S,kps,H", [
    ("sliding", "bf16", 16, 256, 8, "ragged", None, 0, 64),
    ("sliding", "fp8", 16, 256, 3, [600, 511, 4000], None, 0, 32),
    ("full", "f16", 16, 128, 3, [2500, 3, 1200], 3000, 256, 32),
    ("full", "fp8", 16, 256, 2, [2996, 40], 3000, 512, 32),
])
def test_gqa_pieces_consecutive_steps(kind, dtype, G, D, B, pos, S, kps, H):
    spec = gqa_spec(kind, B, dtype, G, D=D, S=S, H=H)
    x = inputs.make_step(spec, positions(kind, B, S, pos, 51), seed=52)
    if kind == "sliding":
        x.pos = np.maximum(x.pos, spec.n_slots).astype(np.int32)
    ring = kind == "sliding"
    kc, vc = x.k_cache.copy(), x.v_cache.copy()
    d = to_dev(x)
    mp = int(x.pos.max()) + 3
    desc = hswd.make_desc(d["k_cache"], n_heads=spec.H, keys_per_split=kps,
                          kv_scale=d["kv_scale"])
    ws = hswd.workspace(desc, ring, mp)
    rng = np.random.default_rng(53)
    for step in range(4):
        if step > 0:
            x.pos = (x.pos + 1).astype(np.int32)
            for f in ("q", "k", "v", "gate"):
                setattr(x, f, rng.standard_normal(getattr(x, f).shape).astype(np.float32))
            # the history this step reads (the parity bar normalises by its V)
            x.k_cache, x.v_cache = kc.copy(), vc.copy()
        ref = oracle.layer_step(x.q, x.k, x.v, x.gate, kc, vc, x.pos, CODE[dtype], ring,
                                spec.rot, spec.theta, write=True, kv_scale=spec.kv_scale)
        say("gqa pieces %s %s G=%d step %d pos=%s" % (kind, dtype, G, step, list(x.pos[:4])))
        out = hswd.layer_step(f32_dev(x.q), f32_dev(x.k), f32_dev(x.v),
                              f32_dev(x.gate), d["k_cache"], d["v_cache"],
                              i32_dev(x.pos), ring, spec.rot, spec.theta, ws, max_pos=mp,
                              desc=desc)
        assert hswd.check_errors(ws) == 0
        assert_parity(out.cpu().numpy(), ref["out"], x, "gqa pieces step %d" % step)
        assert np.array_equal(cache_to_host(d["k_cache"]), kc), "stored keys differ"
        assert np.array_equal(cache_to_host(d["v_cache"]), vc), "stored values differ"


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("fp8", 8)])
def test_gqa_partials_merge_to_oracle(dtype, G):
    """Chunk partials of a grouped full layer (cached keys only), merged by
    hswd_lse_merge, give the oracle's attention over the same keys."""
    B, S = 3, 2500
    spec = gqa_spec("full", B, dtype, G, S=S, H=8 * G // 4 if G == 8 else 8)
    x = inputs.make_step(spec, [2499, 700, 1], seed=31)
    d = to_dev(x)
    hswd.rope_apply(d["q"], d["k"], d["pos"], spec.rot, spec.theta)
    kps = 256 if dtype != "fp8" else 512
    desc = hswd.make_desc(d["k_cache"], n_heads=spec.H, keys_per_split=kps,
                          kv_scale=d["kv_scale"])
    say("gqa partials %s G=%d" % (dtype, G))
    po, pml = hswd.decode_attn_partials(d["q"], d["k_cache"], d["v_cache"], d["pos"], 0,
                                        max_pos=2499, desc=desc)
    merged = hswd.lse_merge(po, pml).cpu().numpy()
    q_rot = d["q"].cpu().numpy().astype(np.float64)
    scale = 1.0 / np.sqrt(spec.D)
    for b in range(B):
        p = int(x.pos[b])
        for h in range(spec.H):
            gk = h // G
            ks = vs = 1.0
            if spec.kv_scale is not None:
                ks, vs = float(spec.kv_scale[0][gk]), float(spec.kv_scale[1][gk])
            m, l, o = oracle.partial(q_rot[b, h], x.k_cache[b, gk], x.v_cache[b, gk],
                                     CODE[dtype], 0, p, scale, ks=ks, vs=vs)
            vmax = np.abs(oracle.decode(CODE[dtype], x.v_cache[b, gk, :p])).max() * vs
            err = np.abs(merged[b, h] - o / l).max() / vmax
            assert err <= 2e-3, (b, h, err)


@pytest.mark.parametrize("kind,G", [("sliding", 4), ("full", 2)])
def test_gqa_equals_repeated_kv_heads(kind, G):
    """A group of G query heads over one kv head gives what G separate heads
    over G copies of that kv head give (H = Hkv): grouping only shares the
    reads.  Within the parity bar (the tile size, and so the online-softmax
    order, differs between the two kernels)."""
    B, S = 6, 2000
    spec = gqa_spec(kind, B, "bf16", G, S=S)
    x = inputs.make_step(spec, positions(kind, B, S, "ragged", 41), seed=42)
    rep = lambda a: np.repeat(a, G, axis=1)
    y = inputs.StepInputs(gqa_spec(kind, B, "bf16", 1, S=S), x.pos, x.q, rep(x.k), rep(x.v),
                          x.gate, rep(x.k_cache), rep(x.v_cache))
    ring = kind == "sliding"
    mp = int(x.pos.max())
    outs = []
    for z in (x, y):
        d = to_dev(z)
        desc = hswd.make_desc(d["k_cache"], n_heads=z.spec.H)
        ws = hswd.workspace(desc, ring, mp)
        say("gqa vs repeated kv %s G=%d Hkv=%d" % (kind, G, z.spec.Hkv))
        outs.append(hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"],
                                    d["v_cache"], d["pos"], ring, z.spec.rot, z.spec.theta, ws,
                                    max_pos=mp, desc=desc).cpu().numpy())
    assert_parity(outs[0], outs[1].astype(np.float64), x, "grouped vs repeated")


def test_gqa_unsupported_is_refused():
    """Grouped layers over a float32 cache or with head_dim 64 have no kernel
    and are refused before any launch."""
    for dtype, D in (("f32", 256), ("bf16", 64)):
        spec = gqa_spec("sliding", 2, dtype, 2, D=D, H=16)
        x = inputs.make_step(spec, [3, 700], seed=51)
        d = to_dev(x)
        desc = hswd.make_desc(d["k_cache"], n_heads=spec.H)
        ws = hswd.workspace(desc, 1, 0)
        with pytest.raises(hswd.HswdError):
            hswd.layer_step(d["q"], d["k"], d["v"], d["gate"], d["k_cache"], d["v_cache"],
                            d["pos"], 1, spec.rot, spec.theta, ws, desc=desc)
