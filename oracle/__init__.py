"""CPU oracle for hybrid sliding-window decode attention -- TEST INFRASTRUCTURE.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  The GPU path never imports it, and it
imports nothing from the GPU path.

The arithmetic lives in `hswd_oracle.c` (plain C, fp64); this module loads it
with ctypes and converts numpy arrays.  Cache element types are passed as
raw bits: float32 arrays for f32, uint16 bit patterns for f16 and bf16,
uint8 codes for fp8 e4m3.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16, FP8 = 0, 1, 2, 3
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16, "fp8": FP8}

_lib = None


def lib(path=None):
    """Load (building if absent) the oracle library; `path` loads a variant."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(L):
    P = ctypes.c_void_p
    i32, f64, sz = ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f16_value.restype = f64
    L.orc_f16_value.argtypes = [ctypes.c_uint16]
    L.orc_bf16_value.restype = f64
    L.orc_bf16_value.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_fp8.restype = ctypes.c_uint8
    L.orc_f32_to_fp8.argtypes = [ctypes.c_float]
    L.orc_fp8_value.restype = f64
    L.orc_fp8_value.argtypes = [ctypes.c_uint8]
    L.orc_round_f32_to.argtypes = [i32, P, sz, P]
    L.orc_decode.argtypes = [i32, P, sz, P]
    L.orc_slot_mask.argtypes = [i32, i32, i32, P, P, P]
    L.orc_rope.argtypes = [P, P, i32, i32, f64, ctypes.c_int64, i32]
    L.orc_rope_batch.argtypes = [P, P, i32, i32, i32, i32, f64, P, i32]
    L.orc_attend.argtypes = [P, P, P, P, i32, i32, i32, P, P, f64, f64, f64]
    L.orc_partial.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f64, f64, f64]
    L.orc_merge.argtypes = [P, P, P, P, i32, i32]
    L.orc_attend_split.argtypes = [P, P, P, P, i32, P, i32, i32, P, P, f64, f64, f64]
    L.orc_sigmoid.restype = f64
    L.orc_sigmoid.argtypes = [f64]
    L.orc_head_gate.argtypes = [P, P, P, i32, i32, i32]
    L.orc_layer_step.restype = i32
    L.orc_layer_step.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, f64, f64, i32,
                                 P, P, P, P, P, P, P, i32, P, P, P, P, P, P, P]
    L.orc_attend_block.argtypes = [P, P, P, P, i32, i32, i32, P, P, f64, f64, f64]
    L.orc_gate_proj.argtypes = [P, P, P, i32, i32, i32]
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def storage_dtype(dtype):
    """numpy container for a cache element type's bits."""
    return {F32: np.float32, FP8: np.uint8}.get(dtype, np.uint16)


# --------------------------------------------------------------------------
# element conversions
# --------------------------------------------------------------------------
def round_to(dtype, x, L=None):
    """float32 -> cache element type bits (round to nearest, ties to even)."""
    L = L or lib()
    x = _c(x, np.float32)
    out = np.empty(x.shape, storage_dtype(dtype))
    L.orc_round_f32_to(dtype, _p(x), x.size, _p(out))
    return out


def decode(dtype, x, L=None):
    """Cache element type bits -> exact float64 values."""
    L = L or lib()
    x = _c(x, storage_dtype(dtype))
    out = np.empty(x.shape, np.float64)
    L.orc_decode(dtype, _p(x), x.size, _p(out))
    return out


# --------------------------------------------------------------------------
# the steps of one layer
# --------------------------------------------------------------------------
def slot_mask(pos, n_slots, ring, L=None):
    L = L or lib()
    pos = _c(pos, np.int32)
    B = pos.size
    slot = np.empty(B, np.int32)
    mask = np.empty((B, n_slots), np.uint8)
    L.orc_slot_mask(B, n_slots, int(ring), _p(pos), _p(slot), _p(mask))
    return slot, mask


def rope(x, pos, rot, theta, interleaved=False, L=None):
    """x [..., n_heads, D] float32 with pos broadcast over the head axis."""
    L = L or lib()
    x = _c(x, np.float32)
    D = x.shape[-1]
    nh = x.shape[-2]
    n = x.size // D
    pos = _c(np.broadcast_to(pos, (n // nh,)), np.int32)
    out = np.empty(x.shape, np.float64)
    L.orc_rope_batch(_p(out), _p(x), n, nh, D, rot, theta, _p(pos), int(interleaved))
    return out


def attend(q, kc, vc, dtype, n, k_new, v_new, scale, ks=1.0, vs=1.0, L=None):
    """One query over rows 0..n-1 of a (rows, D) cache block plus the new entry
    (cached values are ks * decode(K), vs * decode(V))."""
    L = L or lib()
    q = _c(q, np.float64)
    D = q.size
    kc = _c(kc, storage_dtype(dtype))
    vc = _c(vc, storage_dtype(dtype))
    assert kc.size >= n * D and vc.size >= n * D
    o = np.empty(D, np.float64)
    L.orc_attend(_p(o), _p(q), _p(kc), _p(vc), dtype, n, D,
                 _p(_c(k_new, np.float64)), _p(_c(v_new, np.float64)), scale, ks, vs)
    return o


def partial(q, kc, vc, dtype, j0, j1, scale, ks=1.0, vs=1.0, L=None):
    L = L or lib()
    q = _c(q, np.float64)
    D = q.size
    kc = _c(kc, storage_dtype(dtype))
    vc = _c(vc, storage_dtype(dtype))
    m = np.zeros(1)
    l = np.zeros(1)
    o = np.empty(D)
    L.orc_partial(_p(m), _p(l), _p(o), _p(q), _p(kc), _p(vc), dtype, j0, j1, D, scale, ks, vs)
    return m[0], l[0], o


def merge(m, l, o, L=None):
    """Merge partials: m [n], l [n], o [n, D] (o not yet divided by l)."""
    L = L or lib()
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    n, D = o.shape
    out = np.empty(D)
    L.orc_merge(_p(out), _p(m), _p(l), _p(o), n, D)
    return out


def attend_split(q, kc, vc, dtype, bounds, k_new, v_new, scale, ks=1.0, vs=1.0, L=None):
    L = L or lib()
    q = _c(q, np.float64)
    D = q.size
    bounds = _c(bounds, np.int32)
    o = np.empty(D)
    L.orc_attend_split(_p(o), _p(q), _p(_c(kc, storage_dtype(dtype))),
                       _p(_c(vc, storage_dtype(dtype))), dtype, _p(bounds),
                       bounds.size - 1, D, _p(_c(k_new, np.float64)),
                       _p(_c(v_new, np.float64)), scale, ks, vs)
    return o


def sigmoid(g, L=None):
    L = L or lib()
    return L.orc_sigmoid(float(g))


def head_gate(o, g, L=None):
    """o [B, H, D] float64, g [B, H] float32 logits."""
    L = L or lib()
    o = _c(o, np.float64)
    g = _c(g, np.float32)
    B, H, D = o.shape
    out = np.empty_like(o)
    L.orc_head_gate(_p(out), _p(o), _p(g), B, H, D)
    return out


def gate_proj(x, w, L=None):
    """Gate logits [B, H] = x [B, hidden] . w[H, hidden]^T, in fp64."""
    L = L or lib()
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    B, hidden = x.shape
    H = w.shape[0]
    out = np.empty((B, H))
    L.orc_gate_proj(_p(out), _p(x), _p(w), B, hidden, H)
    return out


def layer_step(q, k, v, gate, k_cache, v_cache, pos, dtype, ring, rot, theta,
               scale=None, interleaved=False, write=True, kv_scale=None, L=None):
    """One layer step (rotate, round, attend, gate, write) on host arrays.

    q [B,H,D], k/v [B,Hkv,D] float32; gate [B,H] float32 or None;
    k_cache/v_cache [B,Hkv,n_slots,D] bits of `dtype`, updated in place when
    `write`; pos [B] int32; kv_scale [2, Hkv] float32 per-head scales (K
    then V) or None.  Returns a dict of outputs and the status code.
    """
    L = L or lib()
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    B, H, D = q.shape
    Hkv = k.shape[1]
    n_slots = k_cache.shape[2]
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == storage_dtype(dtype) and v_cache.dtype == storage_dtype(dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = _c(pos, np.int32)
    out = np.empty((B, H, D))
    o_pre = np.empty((B, H, D))
    q_rot = np.empty((B, H, D))
    k_rot32 = np.empty((B, Hkv, D), np.float32)
    k_hat = np.empty((B, Hkv, D), storage_dtype(dtype))
    v_hat = np.empty((B, Hkv, D), storage_dtype(dtype))
    g = None if gate is None else _c(gate, np.float32)
    ksc = None if kv_scale is None else _c(kv_scale, np.float32)
    status = L.orc_layer_step(B, H, Hkv, D, n_slots, dtype, int(ring), rot, theta,
                              float(scale), int(interleaved), _p(pos), _p(q), _p(k),
                              _p(v), _p(g), _p(k_cache), _p(v_cache), int(write), _p(ksc),
                              _p(out), _p(o_pre), _p(q_rot), _p(k_rot32), _p(k_hat),
                              _p(v_hat))
    return dict(out=out, o_pre=o_pre, q_rot=q_rot, k_rot32=k_rot32, k_hat=k_hat,
                v_hat=v_hat, status=status)


def attend_block(q_rot, kc, vc, dtype, n, k_hat, v_hat, scale, ks=1.0, vs=1.0, L=None):
    """One (stream, head) of a step from a cache block and the rounded entry."""
    L = L or lib()
    q_rot = _c(q_rot, np.float64)
    D = q_rot.size
    o = np.empty(D)
    L.orc_attend_block(_p(o), _p(q_rot), _p(_c(kc, storage_dtype(dtype))),
                       _p(_c(vc, storage_dtype(dtype))), dtype, n, D,
                       _p(_c(k_hat, storage_dtype(dtype))),
                       _p(_c(v_hat, storage_dtype(dtype))), scale, ks, vs)
    return o
