"""Adversarial numerics of the fp16 probabilities in the matrix-core kernels.

Over f16 and fp8 caches the grouped kernels (4 and 8 query heads per kv
head) round each probability to fp16 for the value product.  The worst case
for that rounding is many keys far below a dominant one: here every wave's
first key of every chunk dominates (its score 24.68 binary orders above the
rest), so every other key of the 131072 has a probability of about
1.25 * 2^-25 against its wave's running maximum -- below fp16's normal range
had it not been scaled -- and the values are either constant per head (the
output must be that constant) or alternate in sign from key to key.  Every
head is checked against the fp64 oracle under the 2e-3 bar (normalised by the
largest attended |V|), and the margin is printed.
"""
import math

import numpy as np
import pytest
import torch

import hybrid_sliding_window_decode_amd as hswd
import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import CODE, TOL, cache_to_dev, say

pytestmark = pytest.mark.gpu

N_KEYS = 131072
D = 128
HKV = 8


def _case(dtype, H, values):
    S = N_KEYS + 1
    scale = 1.0 / math.sqrt(D)
    desc0 = hswd.binding.AttnDesc(1, H, HKV, D, S, CODE[dtype], scale, 0, 0, None)
    K = hswd.num_splits(desc0, 0, N_KEYS)
    chunk = -(-N_KEYS // K)                               # keys per chunk
    kt = 4096 // D                       # keys per wave tile of these kernels (8 loads)
    # dominant keys: the first key of each wave's first tile in every chunk
    dom = np.zeros(N_KEYS, bool)
    for c0 in range(0, N_KEYS, chunk):
        dom[c0:c0 + 4 * kt:kt] = True
    c = 16.0
    a = 24.678 * math.log(2.0) / (scale * c)            # dominant score - rest = 24.678 bits
    k = np.zeros((1, HKV, S, D), np.float32)
    k[0, :, :N_KEYS, 0] = np.where(dom, c, 0.0)
    v = np.zeros((1, HKV, S, D), np.float32)
    g = np.arange(HKV, dtype=np.float32)[:, None, None]
    if values == "constant":
        v[0, :, :N_KEYS, :] = 1.0 + g / 8.0
    else:
        sign = np.where(np.arange(N_KEYS) % 2 == 0, 1.0, -1.0).astype(np.float32)
        v[0, :, :N_KEYS, :] = sign[None, :, None] * (1.0 + g / 8.0)
        v[0, :, np.nonzero(dom)[0], :] = 0.5
    kc = inputs.cast_bits(k, dtype)
    vc = inputs.cast_bits(v, dtype)
    q = np.zeros((1, H, D), np.float32)
    q[0, :, 0] = a
    k_new = np.zeros((1, HKV, D), np.float32)              # scores 0, like the rest
    v_new = (1.0 + np.arange(HKV, dtype=np.float32)[:, None] / 8.0)[None].repeat(D, 2)

    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    kcd, vcd = cache_to_dev(kc, dtype), cache_to_dev(vc, dtype)
    desc = hswd.make_desc(kcd, n_heads=H)
    ws = hswd.workspace(desc, 0, N_KEYS)
    say("fp16 probabilities: %s H=%d Hkv=%d, %d keys in chunks of %d, values %s" % (
        dtype, H, HKV, N_KEYS, chunk, values))
    out = hswd.decode_attn_full(dev(q), dev(k_new), dev(v_new), kcd, vcd,
                                torch.tensor([N_KEYS], dtype=torch.int32, device="cuda"),
                                N_KEYS, ws, desc=desc).cpu().numpy()
    code = CODE[dtype]
    k_hat = oracle.round_to(code, k_new)
    v_hat = oracle.round_to(code, v_new)
    G = H // HKV
    worst = 0.0
    for h in range(H):
        gg = h // G
        ref = oracle.attend_block(q[0, h].astype(np.float64), kc[0, gg], vc[0, gg], code, N_KEYS,
                                  k_hat[0, gg], v_hat[0, gg], scale)
        vmax = max(float(np.abs(oracle.decode(code, vc[0, gg, :N_KEYS])).max()),
                   float(np.abs(v_new[0, gg]).max()))
        err = float(np.abs(out[0, h] - ref).max()) / vmax
        if values == "constant":
            assert np.allclose(ref, 1.0 + gg / 8.0, rtol=1e-9, atol=0)   # fp64 sums of 2^17 terms
        worst = max(worst, err)
        assert err <= TOL[dtype], (h, err)
    say("  worst normalised error %.3e, bar %.0e (margin x%.0f)" % (
        worst, TOL[dtype], TOL[dtype] / max(worst, 1e-30)))


@pytest.mark.parametrize("values", ["constant", "alternating"])
@pytest.mark.parametrize("dtype,H", [("f16", 32), ("f16", 64), ("fp8", 32), ("fp8", 64)])
def test_dominant_keys_with_tiny_probabilities_131072(dtype, H, values):
    _case(dtype, H, values)
