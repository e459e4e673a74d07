"""Helpers of the GPU parity tests: host <-> device copies of the seeded
inputs and the tolerance checks the parity bar uses.

Tolerances (max over head dims, per (stream, head)):
  f32 caches:        max|gpu - oracle| / max|oracle|          <= 1e-5
  f16 / bf16 caches: max|gpu - oracle| / max|V over attended| <= 2e-3
Slots, masks and stored cache entries: bit-exact.
"""
import sys

import numpy as np
import torch

import oracle

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.float8_e4m3fn}
CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "fp8": 2e-3}


def say(*a):
    """Print and flush: names the case before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def cache_to_dev(bits, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, np.float32)).cuda()
    if dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(bits, np.uint8)).cuda()
        return t.view(torch.float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda()
    return t.view(TORCH_DT[dtype])


def cache_to_host(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def to_dev(x):
    """numpy StepInputs -> dict of device tensors (kv_scale for fp8 caches)."""
    d = dict(q=f32_dev(x.q), k=f32_dev(x.k), v=f32_dev(x.v), gate=f32_dev(x.gate),
             pos=i32_dev(x.pos), k_cache=cache_to_dev(x.k_cache, x.spec.dtype),
             v_cache=cache_to_dev(x.v_cache, x.spec.dtype), kv_scale=None)
    if x.spec.kv_scale is not None:
        d["kv_scale"] = f32_dev(x.spec.kv_scale)
    return d


def entry_codes(x_f32, dtype, scale=None):
    """The oracle's stored code of float32 entries (fp8: of x / scale, the
    quotient rounded to float32)."""
    x = np.asarray(x_f32, np.float32)
    if scale is not None:
        x = (x.astype(np.float64) / np.asarray(scale, np.float64)).astype(np.float32)
    return oracle.round_to(CODE[dtype], x)


def vmax_attended(x):
    """max |V| over the rows each (stream, kv head) attends, plus the new v."""
    vc = oracle.decode(CODE[x.spec.dtype], x.v_cache)
    if x.spec.kv_scale is not None:
        vc = vc * x.spec.kv_scale[1][None, :, None, None]
    S = x.spec.n_slots
    out = np.zeros((x.spec.B, x.spec.Hkv))
    for b, p in enumerate(x.pos):
        n = min(max(int(p), 0), S)
        rows = np.abs(vc[b, :, :n]).max(axis=(1, 2)) if n else np.zeros(x.spec.Hkv)
        out[b] = np.maximum(rows, np.abs(x.v[b]).max(axis=1))
    return out


def rel_err(gpu, ref, x):
    """Per (stream, head) error under the parity bar's normalisation."""
    gpu = np.asarray(gpu, np.float64)
    diff = np.abs(gpu - ref).max(axis=2)
    if x.spec.dtype == "f32":
        den = np.abs(ref).max(axis=2)
    else:
        G = x.spec.H // x.spec.Hkv
        den = np.repeat(vmax_attended(x), G, axis=1)
    return diff / np.maximum(den, 1e-30)


def assert_parity(gpu, ref, x, what=""):
    e = rel_err(gpu, ref, x)
    assert np.all(np.isfinite(np.asarray(gpu))), "non-finite GPU output " + what
    worst = float(e.max())
    say("  %s max normalised error %.3e (bar %.0e)" % (what, worst, TOL[x.spec.dtype]))
    assert worst <= TOL[x.spec.dtype], (what, worst)
    return worst
