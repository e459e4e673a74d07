"""Seeded synthetic inputs for the decode step.

This module only draws numbers: it holds none of the attention arithmetic, and
both the GPU path's tests and the oracle's tests take their inputs from it.

Recipe (the pages measure on-device model runs whose weights are not
available; seeded N(0, 1) data of the same shapes stands in for them):
  * q [B,H,D], k and v [B,Hkv,D], gate logits [B,H]: float32 N(0,1);
  * cache contents: float32 N(0,1), rounded to the cache element type with a
    library cast (numpy float16 / torch bfloat16, both round to nearest even);
  * slots never written are filled with NaN, so any read of them shows up in
    the output.  A ring of n_slots that has seen `pos` tokens has written the
    slots {t mod n_slots : t < pos}; an append cache has written rows < pos.
Small cases draw on the CPU with numpy's default_rng(seed); the full-size
workloads draw on the GPU with a seeded torch generator (Philox), in chunks.
"""
from dataclasses import dataclass, field

import numpy as np

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}


@dataclass
class LayerSpec:
    """One attention layer of a decode step."""
    kind: str                 # "sliding" (ring) or "full" (append cache)
    B: int
    H: int = 8
    Hkv: int = 8
    D: int = 256
    n_slots: int = 511        # ring slots, or append capacity
    dtype: str = "bf16"
    rot: int = 256
    theta: float = 1e4
    kv_scale: object = None   # fp8: float32 [2, Hkv] per-head scales (K then V)


def default_fp8_scales(Hkv):
    """Per-head scales of an fp8 cache: different for every head and for K
    and V, sized so N(0,1) data sits well inside the e4m3 range (+-448)."""
    g = np.arange(Hkv, dtype=np.float32)
    return np.stack([(1 + g / 8) / 64, (1 + g / 4) / 64]).astype(np.float32)


def sliding_spec(B, dtype="bf16", H=8, Hkv=8, D=256, n_slots=511):
    """Sliding layer: 511-slot ring, all head dims rotated at theta 1e4."""
    return LayerSpec("sliding", B, H, Hkv, D, n_slots, dtype, rot=D, theta=1e4,
                     kv_scale=default_fp8_scales(Hkv) if dtype == "fp8" else None)


def full_spec(B, capacity, dtype="bf16", H=8, Hkv=8, D=256):
    """Full layer: append cache, first quarter of the head dims at theta 5e6."""
    return LayerSpec("full", B, H, Hkv, D, capacity, dtype, rot=D // 4, theta=5e6,
                     kv_scale=default_fp8_scales(Hkv) if dtype == "fp8" else None)


def written_rows(kind, n_slots, pos):
    """Boolean [n_slots]: which rows a cache that has seen `pos` tokens holds."""
    s = np.arange(n_slots)
    if kind == "sliding":
        return (s < pos) | (pos >= n_slots)
    return s < pos


def cast_bits(x32, dtype, scale=None):
    """float32 array -> storage bits of `dtype` by a library cast.  fp8: the
    code of x / scale (scale broadcast against x), clamped to +-448 first so
    the cast saturates."""
    if dtype == "fp8":
        import torch
        y = np.ascontiguousarray(x32, np.float32)
        if scale is not None:
            y = (y / np.asarray(scale, np.float32)).astype(np.float32)
        t = torch.from_numpy(np.clip(y, -448.0, 448.0).astype(np.float32))
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    if dtype == "f32":
        return np.ascontiguousarray(x32, np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16)).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def nan_bits(dtype):
    return {"f32": np.float32(np.nan), "f16": np.uint16(0x7e00),
            "bf16": np.uint16(0x7fc0), "fp8": np.uint8(0x7f)}[dtype]


@dataclass
class StepInputs:
    spec: LayerSpec
    pos: np.ndarray           # int32 [B]
    q: np.ndarray             # float32 [B,H,D]
    k: np.ndarray             # float32 [B,Hkv,D]
    v: np.ndarray             # float32 [B,Hkv,D]
    gate: np.ndarray          # float32 [B,H]
    k_cache: np.ndarray       # bits [B,Hkv,n_slots,D]
    v_cache: np.ndarray
    extra: dict = field(default_factory=dict)


def make_step(spec, pos, seed, poison=True):
    """Host (numpy) inputs of one layer step for streams at positions `pos`."""
    rng = np.random.default_rng(seed)
    pos = np.array(np.broadcast_to(np.asarray(pos, np.int32), (spec.B,)), np.int32)
    B, H, Hkv, D, S = spec.B, spec.H, spec.Hkv, spec.D, spec.n_slots
    q = rng.standard_normal((B, H, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    gate = rng.standard_normal((B, H), dtype=np.float32)
    ks = vs = None
    if spec.dtype == "fp8":
        ks = spec.kv_scale[0][None, :, None, None]
        vs = spec.kv_scale[1][None, :, None, None]
    kc = cast_bits(rng.standard_normal((B, Hkv, S, D), dtype=np.float32), spec.dtype, ks)
    vc = cast_bits(rng.standard_normal((B, Hkv, S, D), dtype=np.float32), spec.dtype, vs)
    if poison:
        for b in range(B):
            dead = ~written_rows(spec.kind, S, int(pos[b]))
            kc[b][:, dead, :] = nan_bits(spec.dtype)
            vc[b][:, dead, :] = nan_bits(spec.dtype)
    return StepInputs(spec, pos, q, k, v, gate, kc, vc)


def gate_inputs(B, hidden, H, seed):
    """Post-norm layer input x [B, hidden] ~ N(0,1) and gate weight
    w_g [H, hidden] ~ N(0, 1/hidden) (float32), so logits are ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, hidden), dtype=np.float32)
    w = (rng.standard_normal((H, hidden), dtype=np.float32) / np.float32(np.sqrt(hidden)))
    return x, w.astype(np.float32)


def ragged_positions(B, lo, hi, seed):
    """Integer positions uniform in [lo, hi], seeded."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


# ----------------------------------------------------------------------------
# Named workloads.  Sizes follow the workloads the pages' model implies: 8
# heads of 256 dims, a 511-slot ring, 3 sliding layers per full layer.
# ----------------------------------------------------------------------------
WORKLOADS = {
    # 1 stream, one sliding layer, fp32 ring at position 600 (wrapped)
    "sliding_1x600_f32": dict(kind="sliding", B=1, dtype="f32", pos=600, seed=1),
    # 1 stream, one full layer, context 1024, fp16 cache
    "full_1x1024_f16": dict(kind="full", B=1, dtype="f16", pos=1024, seed=2),
    # 64 streams, one sliding layer, ragged positions in [1, 4096], bf16 ring
    "sliding_64xragged_bf16": dict(kind="sliding", B=64, dtype="bf16", pos="ragged", seed=3),
    # 28-layer step (21 sliding + 7 full), 64 streams at context 4096, bf16
    "step28_64x4096_bf16": dict(kind="step", B=64, dtype="bf16", pos=4096, seed=4, layers=28),
    # 8 streams at context 131072, full and sliding layers, bf16
    "long_8x131072_bf16": dict(kind="long", B=8, dtype="bf16", pos=131072, seed=5),
}


def layer_is_full(l):
    """3:1 interleave: layer l is full attention iff l % 4 == 3."""
    return l % 4 == 3


# ----------------------------------------------------------------------------
# Device-side generation for the full-size workloads (torch, seeded Philox).
# ----------------------------------------------------------------------------
def device_normal_(t, gen, chunk_rows=1 << 16, scale=None):
    """Fill a CUDA tensor of any float dtype with N(0,1) drawn in float32.
    fp8 tensors [B, Hkv, S, D] get the code of x / scale[g] (clamped to
    +-448), scale a float32 [Hkv] array."""
    import torch
    if t.dtype == torch.float8_e4m3fn:
        sc = torch.as_tensor(np.asarray(scale, np.float32), device=t.device)
        for b in range(t.shape[0]):
            for g in range(t.shape[1]):
                x = torch.randn(t.shape[2] * t.shape[3], generator=gen, device=t.device,
                                dtype=torch.float32)
                t[b, g].view(-1)[:] = (x / sc[g]).clamp(-448.0, 448.0).to(t.dtype)
        return t
    flat = t.view(-1)
    n = flat.numel()
    step = chunk_rows * 256
    for i in range(0, n, step):
        j = min(n, i + step)
        flat[i:j] = torch.randn(j - i, generator=gen, device=t.device,
                                dtype=torch.float32).to(t.dtype)
    return t


def device_step(spec, pos, seed, device="cuda"):
    """Device tensors of one layer step (torch), for the full-size workloads.

    Caches are drawn N(0,1) in float32 then cast to the element type; rows
    never written are NaN-poisoned per stream.  Returns a dict of tensors.
    """
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "fp8": torch.float8_e4m3fn}[spec.dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    B, H, Hkv, D, S = spec.B, spec.H, spec.Hkv, spec.D, spec.n_slots
    pos_t = torch.as_tensor(np.broadcast_to(np.asarray(pos, np.int32), (B,)).copy(),
                            dtype=torch.int32)
    q = torch.randn(B, H, D, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(B, Hkv, D, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(B, Hkv, D, generator=gen, device=device, dtype=torch.float32)
    gate = torch.randn(B, H, generator=gen, device=device, dtype=torch.float32)
    kc = torch.empty(B, Hkv, S, D, device=device, dtype=tdt)
    vc = torch.empty(B, Hkv, S, D, device=device, dtype=tdt)
    fp8 = spec.dtype == "fp8"
    device_normal_(kc, gen, scale=spec.kv_scale[0] if fp8 else None)
    device_normal_(vc, gen, scale=spec.kv_scale[1] if fp8 else None)
    for b in range(B):
        dead = torch.from_numpy(~written_rows(spec.kind, S, int(pos_t[b])))
        if bool(dead.any()):
            idx = dead.nonzero().view(-1).to(device)
            if fp8:                                   # NaN code 0x7f
                kc[b].view(torch.uint8).index_fill_(1, idx, 0x7f)
                vc[b].view(torch.uint8).index_fill_(1, idx, 0x7f)
            else:
                kc[b].index_fill_(1, idx, float("nan"))
                vc[b].index_fill_(1, idx, float("nan"))
    out = dict(pos=pos_t.to(device), q=q, k=k, v=v, gate=gate, k_cache=kc, v_cache=vc)
    if fp8:
        out["kv_scale"] = torch.as_tensor(spec.kv_scale, device=device)
    return out
