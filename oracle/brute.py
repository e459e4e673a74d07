"""Brute-force windowed decode attention over a full token history.

TEST INFRASTRUCTURE.  A second, independent statement of what a decode step
computes, used to pin the ring oracle on tiny cases: it never forms a ring or
a slot.  At step p it attends over the raw history of positions
max(0, p - window + 1) .. p, each key rotated at its own position, in plain
Python floats (complex rotation from the textbook form of RoPE: the pair
(x_i, x_{i+rot/2}) is the complex number x_i + j x_{i+rot/2}, turned by
exp(j * t * theta^(-2i/rot))).

Sources: vLLM-Omni fork commit log, the score-space join commit (a 512-token
window counts the current token, so the cache holds 511 earlier keys) and the
Spark-X2.5 model commit (per-layer-type RoPE, sigmoid head gate).

Rounding of stored entries to the cache element type uses library casts
(struct float32 packing, numpy float16, torch bfloat16); the oracle's own
converter is pinned against the same casts.
"""
import cmath
import math
import struct

import numpy as np


def to_f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def round_elt(x, dtype, scale=1.0):
    """float (already a float32 value) -> the value the cache type stores
    (fp8: scale * e4m3 code of the float32 quotient x / scale, saturated)."""
    x = to_f32(x)
    if dtype == "fp8":
        import torch
        y = torch.tensor([x], dtype=torch.float32) / torch.tensor([scale], dtype=torch.float32)
        c = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).float()[0]
        return float(c) * float(np.float32(scale))
    if dtype == "f32":
        return x
    if dtype == "f16":
        return float(np.float32(x).astype(np.float16))
    if dtype == "bf16":
        import torch
        return float(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).float()[0])
    raise ValueError(dtype)


def rotate(x, t, rot, theta):
    """RoPE of one vector (list of floats) at position t, rotate-half pairs."""
    out = list(x)
    half = rot // 2
    for i in range(half):
        z = complex(x[i], x[i + half]) * cmath.exp(1j * t * theta ** (-2.0 * i / rot))
        out[i], out[i + half] = z.real, z.imag
    return out


def step(history, p, window, H, Hkv, rot, theta, dtype, scale, gate=None, kv_scale=None):
    """Output of step p: history[t] = (q [H][D], k [Hkv][D], v [Hkv][D]).

    window = number of positions attended including the current one
    (None for a full-attention layer); kv_scale = per-head (K, V) scales of
    an fp8 cache, [2][Hkv].  Returns out[h][d] as floats.
    """
    q, _, _ = history[p]
    first = 0 if window is None else max(0, p - window + 1)
    G = H // Hkv
    out = []
    for h in range(H):
        g = h // G
        qr = rotate(q[h], p, rot, theta)
        scores, vals = [], []
        for t in range(first, p + 1):
            _, kt, vt = history[t]
            ks = 1.0 if kv_scale is None else kv_scale[0][g]
            vs = 1.0 if kv_scale is None else kv_scale[1][g]
            kr = [round_elt(to_f32(x), dtype, ks) for x in rotate(kt[g], t, rot, theta)]
            vr = [round_elt(x, dtype, vs) for x in vt[g]]
            scores.append(scale * math.fsum(a * b for a, b in zip(qr, kr)))
            vals.append(vr)
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        tot = math.fsum(w)
        o = [math.fsum(wi * vi[d] for wi, vi in zip(w, vals)) / tot for d in range(len(qr))]
        if gate is not None:
            sg = 1.0 / (1.0 + math.exp(-gate[h]))
            o = [x * sg for x in o]
        out.append(o)
    return out
