"""Pins of the CPU oracle: checks against facts fixed by the pages and by
mathematics, each a function of an oracle library handle `L`, so that the
mutant tests can run the same pins against planted mistakes.

Every pin raises AssertionError when the oracle disagrees with the fact it
checks.  Sources are cited per pin; "score-space join commit", "Spark-X2.5
model commit" and "per-layer-type KV export commit" are commits in the
vLLM-Omni fork commit log (tea.kyle-merritt.com, anodyine/vllm-omni);
"TensorFold #608" is the review thread of TensorFold pull request 608.
"""
import itertools
import math

import numpy as np

import oracle
from oracle import brute
from hybrid_sliding_window_decode_amd import inputs

F32, F16, BF16, FP8 = oracle.F32, oracle.F16, oracle.BF16, oracle.FP8
NAMES = {F32: "f32", F16: "f16", BF16: "bf16", FP8: "fp8"}


def _torch_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _nan_bits(dtype):
    return {F32: np.float32(np.nan), F16: np.uint16(0x7e00), BF16: np.uint16(0x7fc0),
            FP8: np.uint8(0x7f)}[dtype]


# ----------------------------------------------------------------------------
# rounding to the cache element type (IEEE round to nearest, ties to even)
# ----------------------------------------------------------------------------
def rne_special_inputs():
    """float32 inputs at every tie and edge of the float16 and bfloat16 grids:
    midpoints between all adjacent finite values (exact in float32), the
    float32 neighbours of each midpoint, and the grid values themselves."""
    h = np.arange(0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid16 = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    b = (np.arange(0x7f80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    mid_b = ((b[:-1] + b[1:]) / 2).astype(np.float32)
    top16 = np.float32(65520.0)
    topb = np.float32(np.ldexp(2.0 - 2.0 ** -8, 127))
    core = np.concatenate([mid16, mid_b, h.astype(np.float32), b.astype(np.float32),
                           [top16, topb, np.float32(2.0 ** -25), np.float32(2.0 ** -133)]])
    core = core.astype(np.float32)
    up = np.nextafter(core, np.float32(np.inf))
    dn = np.nextafter(core, np.float32(0))
    allv = np.concatenate([core, up, dn])
    return np.concatenate([allv, -allv]).astype(np.float32)


def check_rne(L, x):
    """Oracle rounding of float32 x to f16 / bf16 vs numpy / torch casts."""
    x = np.ascontiguousarray(x, np.float32)
    nan = np.isnan(x)
    f16 = oracle.round_to(F16, x, L)
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).view(np.uint16)
    bad = (~nan) & (f16 != ref16)
    assert not bad.any(), "f16 rounding differs at %s" % hex(int(x.view(np.uint32)[bad][0]))
    bf = oracle.round_to(BF16, x, L)
    refb = _torch_bf16_bits(x)
    bad = (~nan) & (bf != refb)
    assert not bad.any(), "bf16 rounding differs at %s" % hex(int(x.view(np.uint32)[bad][0]))
    if nan.any():
        # NaN payload rules differ between libraries; the fact checked is
        # that NaN stays NaN with its sign.
        s = (x.view(np.uint32)[nan] >> 31).astype(np.uint16)
        h = f16[nan]
        assert ((h & 0x7c00) == 0x7c00).all() and ((h & 0x3ff) != 0).all()
        assert ((h >> 15) == s).all()
        g = bf[nan]
        assert ((g & 0x7f80) == 0x7f80).all() and ((g & 0x7f) != 0).all()
        assert ((g >> 15) == s).all()


def pin_rne_quick(L):
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    check_rne(L, np.concatenate([u.view(np.float32), rne_special_inputs()]))


def fp8_special_inputs():
    """float32 inputs at every tie and edge of the e4m3 grid, their float32
    neighbours, and out-of-range values."""
    import torch
    codes = torch.arange(0x7f, dtype=torch.int32).to(torch.uint8)      # 0 .. 448
    v = codes.view(torch.float8_e4m3fn).double().numpy()
    mids = (v[:-1] + v[1:]) / 2
    core = np.concatenate([v, mids, [464.0, 465.0, 480.0, 500.0, 1e6, 2.0 ** -10,
                                     3 * 2.0 ** -11]]).astype(np.float32)
    allv = np.concatenate([core, np.nextafter(core, np.float32(np.inf)),
                           np.nextafter(core, np.float32(0)), [np.inf]])
    return np.concatenate([allv, -allv]).astype(np.float32)


def pin_fp8_codec(L):
    """OCP e4m3: all 256 codes decode to torch's float8_e4m3fn values; the
    saturating round-to-nearest-even encoder equals torch's cast of the input
    clamped to +-448, on every tie and edge and on 2^20 random patterns."""
    import torch
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    d = oracle.decode(FP8, codes, L)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(d), np.isnan(ref))
    assert np.array_equal(d[~np.isnan(d)], ref[~np.isnan(ref)])
    rng = np.random.default_rng(33)
    rnd = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.concatenate([fp8_special_inputs(), rnd, rnd * np.float32(1e-37)])
    x = x.astype(np.float32)
    got = oracle.round_to(FP8, x, L)
    nan = np.isnan(x)
    want = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8)
    want = want.numpy()
    bad = (~nan) & (got != want)
    assert not bad.any(), "fp8 rounding differs at %r" % x[bad][:4]
    assert np.all((got[nan] & 0x7f) == 0x7f)
    assert np.all((got[nan] >> 7) == (x[nan].view(np.uint32) >> 31))


def pin_decode(L):
    """Exact values of every float16 / bfloat16 bit pattern vs library casts."""
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    d16 = oracle.decode(F16, allh, L)
    ref = allh.view(np.float16).astype(np.float64)
    same = (d16 == ref) | (np.isnan(d16) & np.isnan(ref))
    assert same.all()
    import torch
    db = oracle.decode(BF16, allh, L)
    refb = torch.from_numpy(allh.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    same = (db == refb) | (np.isnan(db) & np.isnan(refb))
    assert same.all()


# ----------------------------------------------------------------------------
# RoPE (Spark-X2.5 model commit: sliding layers all 256 dims at theta 1e4,
# full layers the first quarter at theta 5e6)
# ----------------------------------------------------------------------------
def pin_rope(L):
    rng = np.random.default_rng(5)
    D = 256
    for rot, theta in [(256, 1e4), (64, 5e6), (16, 1e4)]:
        x = rng.standard_normal((4, 2, D)).astype(np.float32)
        pos = np.array([0, 1, 600, 131072], np.int32)
        out = oracle.rope(x, pos, rot, theta, L=L)
        x64 = x.astype(np.float64)
        # position 0 is the identity, bit for bit
        assert np.array_equal(out[0], x64[0])
        # dims at or past the rotary width are untouched
        assert np.array_equal(out[..., rot:], x64[..., rot:])
        # textbook complex form: (x_i + j x_{i+rot/2}) * exp(j * pos * theta^(-2i/rot))
        half = rot // 2
        z = x64[..., :half] + 1j * x64[..., half:rot]
        inv = theta ** (-2.0 * np.arange(half) / rot)
        zr = z * np.exp(1j * pos[:, None, None].astype(np.float64) * inv)
        # both sides form the fp64 angle pos*inv_i, which may differ by an ulp
        # of the angle (1.5e-11 rad at 1e5 rad): allow a few ulps per position
        tol = (1e-14 * (1.0 + pos.astype(np.float64)))[:, None, None]
        assert np.all(np.abs(out[..., :half] - zr.real) < tol)
        assert np.all(np.abs(out[..., half:rot] - zr.imag) < tol)
        # pair norms are preserved
        n0 = x64[..., :half] ** 2 + x64[..., half:rot] ** 2
        n1 = out[..., :half] ** 2 + out[..., half:rot] ** 2
        assert np.max(np.abs(n0 - n1) / np.maximum(n0, 1e-30)) < 1e-12
    # relative position: <rope(q,p), rope(k,t)> == <rope(q,p-t), k> on rotated dims
    for rot, theta in [(256, 1e4), (64, 5e6)]:
        q = rng.standard_normal((1, 1, D)).astype(np.float32)
        k = rng.standard_normal((1, 1, D)).astype(np.float32)
        for p, t in [(600, 89), (4096, 4000), (37, 37)]:
            a = np.dot(oracle.rope(q, [p], rot, theta, L=L)[0, 0, :rot],
                       oracle.rope(k, [t], rot, theta, L=L)[0, 0, :rot])
            b = np.dot(oracle.rope(q, [p - t], rot, theta, L=L)[0, 0, :rot],
                       k.astype(np.float64)[0, 0, :rot])
            assert abs(a - b) < 1e-9 * (1 + abs(b))


# ----------------------------------------------------------------------------
# slot and mask (score-space join commit: ring slot t mod 511, unwritten
# slots masked, no reordering)
# ----------------------------------------------------------------------------
def pin_slot_mask(L):
    S = 7
    pos = np.arange(0, 30, dtype=np.int32)
    for ring in (1, 0):
        n_slots = S if ring else 40
        slot, mask = oracle.slot_mask(pos, n_slots, ring, L=L)
        for b, p in enumerate(pos):
            written = np.zeros(n_slots, bool)
            for t in range(int(p)):              # replay the history
                written[t % n_slots if ring else t] = True
            assert np.array_equal(mask[b].astype(bool), written)
            assert slot[b] == (p % n_slots if ring else p)


# ----------------------------------------------------------------------------
# brute force over the raw history, several steps through the ring's wrap
# (score-space join commit: the window counts the current token; the write
# goes to pos mod n_slots and must follow the read)
# ----------------------------------------------------------------------------
def pin_brute_multistep(L):
    cases = [("sliding", F32, 2, 2), ("sliding", F16, 4, 2), ("sliding", BF16, 2, 2),
             ("full", F32, 2, 2), ("full", BF16, 4, 2), ("sliding", FP8, 4, 2), ("full", FP8, 2, 2)]
    D, W, steps = 8, 4, 12
    for kind, dt, H, Hkv in cases:
        rng = np.random.default_rng(100 + H + dt)
        ring = kind == "sliding"
        n_slots = W - 1 if ring else steps
        rot, theta = (D, 1e4) if ring else (D // 4, 5e6)
        scale = 1.0 / math.sqrt(D)
        hist = [(rng.standard_normal((H, D)).astype(np.float32),
                 rng.standard_normal((Hkv, D)).astype(np.float32),
                 rng.standard_normal((Hkv, D)).astype(np.float32)) for _ in range(steps)]
        gate = rng.standard_normal(H).astype(np.float32)
        ksc = inputs.default_fp8_scales(Hkv) if dt == FP8 else None
        sd = oracle.storage_dtype(dt)
        kc = np.full((1, Hkv, n_slots, D), _nan_bits(dt), sd)
        vc = np.full((1, Hkv, n_slots, D), _nan_bits(dt), sd)
        hist_py = [(q.tolist(), k.tolist(), v.tolist()) for q, k, v in hist]
        for p in range(steps):
            q, k, v = hist[p]
            r = oracle.layer_step(q[None], k[None], v[None], gate[None], kc, vc, [p], dt,
                                  ring, rot, theta, scale, write=True, kv_scale=ksc, L=L)
            ref = np.array(brute.step(hist_py, p, W if ring else None, H, Hkv, rot, theta,
                                      NAMES[dt], scale, gate.tolist(),
                                      None if ksc is None else ksc.tolist()))
            err = np.max(np.abs(r["out"][0] - ref)) / np.max(np.abs(ref))
            assert err < 1e-12, (kind, NAMES[dt], p, err)


# ----------------------------------------------------------------------------
# closed forms and invariants of the attention step
# ----------------------------------------------------------------------------
def _step_inputs(kind, dt, B, pos, seed, S=None):
    spec = (inputs.sliding_spec(B, NAMES[dt]) if kind == "sliding"
            else inputs.full_spec(B, S or int(np.max(pos)) + 1, NAMES[dt]))
    if S is not None and kind == "sliding":
        spec.n_slots = S
    return inputs.make_step(spec, pos, seed)


def pin_single_key(L):
    """pos 0: only the new entry is attended; its weight is exp(0)=1 and the
    sum of weights is 1, so the output is the rounded value, bit for bit."""
    for kind in ("sliding", "full"):
        for dt in (F32, F16, BF16):
            x = _step_inputs(kind, dt, 2, 0, 21, S=511 if kind == "sliding" else 4)
            r = oracle.layer_step(x.q, x.k, x.v, x.gate, x.k_cache, x.v_cache, x.pos, dt,
                                  kind == "sliding", x.spec.rot, x.spec.theta, write=False, L=L)
            vh = oracle.decode(dt, r["v_hat"], L)
            assert np.array_equal(r["o_pre"], vh)


def pin_equal_scores(L):
    """q = 0: every score is 0, so the output is the plain mean of the
    attended values (valid cached rows and the new entry)."""
    for kind, pos, dt in [("sliding", [300, 600, 1], BF16), ("full", [20, 5, 0], F16),
                          ("sliding", [511, 512, 510], F32)]:
        x = _step_inputs(kind, dt, 3, pos, 22)
        q0 = np.zeros_like(x.q)
        r = oracle.layer_step(q0, x.k, x.v, None, x.k_cache, x.v_cache, x.pos, dt,
                              kind == "sliding", x.spec.rot, x.spec.theta, write=False, L=L)
        vc = oracle.decode(dt, x.v_cache, L)
        vh = oracle.decode(dt, r["v_hat"], L)
        S = x.spec.n_slots
        for b, p in enumerate(x.pos):
            n = min(int(p), S)
            for h in range(x.spec.H):
                rows = np.concatenate([vc[b, h, :n], vh[b, h][None]], 0)
                assert np.max(np.abs(r["o_pre"][b, h] - rows.mean(0))) < 1e-14


def pin_join_equals_concat(L):
    """Score-space join commit: scoring the cache and the new token
    separately and joining the score vectors is the softmax over the key
    matrix with the (rounded) new key appended."""
    for kind, dt, pos in [("sliding", BF16, [700, 200]), ("full", F16, [300, 1])]:
        x = _step_inputs(kind, dt, 2, pos, 23)
        r = oracle.layer_step(x.q, x.k, x.v, None, x.k_cache, x.v_cache, x.pos, dt,
                              kind == "sliding", x.spec.rot, x.spec.theta, write=False, L=L)
        kc = oracle.decode(dt, x.k_cache, L)
        vc = oracle.decode(dt, x.v_cache, L)
        kh = oracle.decode(dt, r["k_hat"], L)
        vh = oracle.decode(dt, r["v_hat"], L)
        for b, p in enumerate(x.pos):
            n = min(int(p), x.spec.n_slots)
            for h in range(x.spec.H):
                K = np.concatenate([kc[b, h, :n], kh[b, h][None]], 0)
                V = np.concatenate([vc[b, h, :n], vh[b, h][None]], 0)
                s = K @ r["q_rot"][b, h] / 16.0
                w = np.exp(s - s.max())
                o = (w[:, None] * V).sum(0) / w.sum()
                assert np.max(np.abs(o - r["o_pre"][b, h])) < 1e-13


def pin_split_invariance(L):
    """TensorFold #608: cutting the key range into chunks and merging the
    partials gives the unsplit result, for every contiguous partition,
    empty chunks included."""
    rng = np.random.default_rng(24)
    D, n = 16, 7
    kc = inputs.cast_bits(rng.standard_normal((n, D)).astype(np.float32), "bf16")
    vc = inputs.cast_bits(rng.standard_normal((n, D)).astype(np.float32), "bf16")
    q = rng.standard_normal(D) * 2
    kn = rng.standard_normal(D)
    vn = rng.standard_normal(D)
    ref = oracle.attend(q, kc, vc, BF16, n, kn, vn, 0.25, L=L)
    for cuts in itertools.product([0, 1], repeat=n - 1):
        bounds = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [n]
        for extra in ([], [0], [n], [3, 3]):
            bd = sorted(bounds + extra)
            o = oracle.attend_split(q, kc, vc, BF16, bd, kn, vn, 0.25, L=L)
            assert np.max(np.abs(o - ref)) < 1e-13, bd


def pin_permutation(L):
    """Score-space join commit: softmax over keys ignores slot order, so any
    permutation of the cached rows gives the same output."""
    rng = np.random.default_rng(25)
    D, n = 256, 60
    kc = inputs.cast_bits(rng.standard_normal((n, D)).astype(np.float32), "f16")
    vc = inputs.cast_bits(rng.standard_normal((n, D)).astype(np.float32), "f16")
    q = rng.standard_normal(D)
    kn, vn = rng.standard_normal(D), rng.standard_normal(D)
    ref = oracle.attend(q, kc, vc, F16, n, kn, vn, 1 / 16, L=L)
    for _ in range(3):
        perm = rng.permutation(n)
        o = oracle.attend(q, kc[perm], vc[perm], F16, n, kn, vn, 1 / 16, L=L)
        assert np.max(np.abs(o - ref)) < 1e-13


def pin_ring_equals_roll(L):
    """Score-space join commit: a ring and the rolled window over the same
    history give the same output.  600 tokens, 511 slots: positions 89..599
    sit at slot t mod 511 in the ring and in order in the rolled copy."""
    rng = np.random.default_rng(26)
    D, S, P = 256, 511, 600
    keys = rng.standard_normal((P, 1, D)).astype(np.float32)
    kr = oracle.rope(keys, np.arange(P, dtype=np.int32), 256, 1e4, L=L)[:, 0]
    kbits = inputs.cast_bits(kr.astype(np.float32), "bf16")
    vbits = inputs.cast_bits(rng.standard_normal((P, D)).astype(np.float32), "bf16")
    ring_k = np.empty((S, D), np.uint16)
    ring_v = np.empty((S, D), np.uint16)
    for t in range(P - S, P):
        ring_k[t % S] = kbits[t]
        ring_v[t % S] = vbits[t]
    q = oracle.rope(rng.standard_normal((1, 1, D)).astype(np.float32), [P], 256, 1e4, L=L)[0, 0]
    kn, vn = rng.standard_normal(D), rng.standard_normal(D)
    a = oracle.attend(q, ring_k, ring_v, BF16, S, kn, vn, 1 / 16, L=L)
    b = oracle.attend(q, kbits[P - S:], vbits[P - S:], BF16, S, kn, vn, 1 / 16, L=L)
    assert np.max(np.abs(a - b)) < 1e-12


def pin_merge(L):
    """Merge of partials: a single partial gives o/l; empty partials
    (m = -inf, l = 0) change nothing and never make NaN; order is free;
    a partial split in two merges back to the whole."""
    rng = np.random.default_rng(27)
    D = 32
    m = rng.standard_normal(5)
    l = rng.uniform(0.5, 3, 5)
    o = rng.standard_normal((5, D))
    one = oracle.merge(m[:1], l[:1], o[:1], L=L)
    assert np.max(np.abs(one - o[0] / l[0])) < 1e-15
    ref = oracle.merge(m, l, o, L=L)
    me = np.concatenate([m, [-np.inf]])
    le = np.concatenate([l, [0.0]])
    oe = np.concatenate([o, np.zeros((1, D))])
    e = oracle.merge(me, le, oe, L=L)
    assert np.all(np.isfinite(e)) and np.max(np.abs(e - ref)) < 1e-14
    perm = rng.permutation(5)
    assert np.max(np.abs(oracle.merge(m[perm], l[perm], o[perm], L=L) - ref)) < 1e-14
    # closed form from the definition of softmax over the union of key sets
    M = m.max()
    w = l * np.exp(m - M)
    direct = (o * np.exp(m - M)[:, None]).sum(0) / w.sum()
    assert np.max(np.abs(direct - ref)) < 1e-14


def pin_gate(L):
    """Spark-X2.5 model commit: the gate scales each head's output by a
    sigmoid.  sigma(0) = 1/2 exactly; sigma saturates to 1 and 0; it agrees
    with scipy's logistic function."""
    from scipy.special import expit
    assert oracle.sigmoid(0.0, L=L) == 0.5
    g = np.linspace(-30, 30, 601)
    s = np.array([oracle.sigmoid(x, L=L) for x in g])
    assert np.max(np.abs(s - expit(g)) / expit(g)) < 1e-14
    rng = np.random.default_rng(28)
    o = rng.standard_normal((2, 3, 8))
    gl = np.array([[0, 40, -40], [1, -1, 0]], np.float32)
    out = oracle.head_gate(o, gl, L=L)
    assert np.array_equal(out[0, 0], o[0, 0] * 0.5)
    assert np.max(np.abs(out[0, 1] - o[0, 1])) < 1e-16 * 8
    assert np.max(np.abs(out[0, 2])) < 1e-17 * 8
    assert np.max(np.abs(out[1, 0] - o[1, 0] * expit(1.0))) < 1e-15


def pin_gate_proj(L):
    """Per-layer-type KV export commit: the gate is [2048, 8], one logit per
    head from the layer's input; against numpy's float64 matmul."""
    x, w = inputs.gate_inputs(5, 2048, 8, seed=31)
    got = oracle.gate_proj(x, w, L=L)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.max(np.abs(got - ref)) < 1e-12 * np.max(np.abs(x)) * np.abs(w).sum(1).max()
    x2, w2 = inputs.gate_inputs(3, 100, 7, seed=32)     # non-square, odd sizes
    assert np.max(np.abs(oracle.gate_proj(x2, w2, L=L) - x2.astype(np.float64) @ w2.T)) < 1e-12


def pin_attend_block(L):
    """The per-(stream, head) entry the full-size checks use equals the
    layer step's pre-gate output for the same head: it takes the rotated
    query, the head's cache block and the stored entry's codes, and must
    decode and scale the entry exactly as the step does (score-space join
    commit: the new token is scored as the entry that is stored).  Every
    cache type, per-head fp8 scales that are not powers of two, a grouped
    head mapping, rings below and past capacity and an append cache."""
    cases = [("sliding", F32, 8, 8, [600, 5]), ("full", F16, 8, 8, [40, 0]),
             ("sliding", BF16, 8, 8, [511, 100]), ("sliding", FP8, 8, 8, [700, 3]),
             ("full", FP8, 8, 4, [30, 1]), ("full", BF16, 8, 2, [17, 64])]
    for kind, dt, H, Hkv, pos in cases:
        ring = kind == "sliding"
        spec = (inputs.sliding_spec(2, NAMES[dt], H=H, Hkv=Hkv, D=128) if ring
                else inputs.full_spec(2, max(pos) + 1, NAMES[dt], H=H, Hkv=Hkv, D=128))
        x = inputs.make_step(spec, pos, 41 + dt)
        ksc = spec.kv_scale
        r = oracle.layer_step(x.q, x.k, x.v, None, x.k_cache, x.v_cache, x.pos, dt, ring,
                              spec.rot, spec.theta, write=False, kv_scale=ksc, L=L)
        G = H // Hkv
        for b, p in enumerate(pos):
            n = min(p, spec.n_slots)
            for h in range(H):
                g = h // G
                ks = 1.0 if ksc is None else float(ksc[0, g])
                vs = 1.0 if ksc is None else float(ksc[1, g])
                o = oracle.attend_block(r["q_rot"][b, h], x.k_cache[b, g], x.v_cache[b, g], dt,
                                        n, r["k_hat"][b, g], r["v_hat"][b, g],
                                        1.0 / math.sqrt(spec.D), ks, vs, L=L)
                ref = r["o_pre"][b, h]
                assert np.max(np.abs(o - ref)) <= 1e-14 * np.max(np.abs(ref)), (
                    kind, NAMES[dt], b, h)


def pin_capacity_and_poison(L):
    """An append position at the capacity is reported (-4) and its write is
    skipped; NaN in unwritten slots never reaches the output."""
    x = _step_inputs("full", BF16, 3, [5, 9, 2], 29, S=10)
    x.pos[1] = 10
    kc0 = x.k_cache.copy()
    r = oracle.layer_step(x.q, x.k, x.v, x.gate, x.k_cache, x.v_cache, x.pos, BF16, 0,
                          64, 5e6, write=True, L=L)
    assert r["status"] == -4
    assert np.array_equal(x.k_cache[1].view(np.uint16), kc0[1].view(np.uint16))
    assert np.all(np.isfinite(r["out"][[0, 2]]))
    y = _step_inputs("sliding", F16, 6, [1, 2, 100, 510, 511, 5000], 30)
    r = oracle.layer_step(y.q, y.k, y.v, y.gate, y.k_cache, y.v_cache, y.pos, F16, 1,
                          256, 1e4, write=True, L=L)
    assert r["status"] == 0 and np.all(np.isfinite(r["out"]))


QUICK_PINS = [pin_rne_quick, pin_fp8_codec, pin_decode, pin_rope, pin_slot_mask, pin_brute_multistep,
              pin_single_key, pin_equal_scores, pin_join_equals_concat,
              pin_split_invariance, pin_permutation, pin_ring_equals_roll, pin_merge,
              pin_gate, pin_gate_proj, pin_attend_block, pin_capacity_and_poison]
