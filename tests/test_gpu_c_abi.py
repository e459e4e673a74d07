"""The C ABI called from C: tests/c_abi/layer_step (no Python, no torch in
it; built by the build entry point) reads one layer step's inputs from raw
files, runs hswd_layer_step through include/hswd.h and writes the output
and both caches back.  Its files are checked against the oracle: the
output under the parity bar, both caches bit for bit against the oracle's
(its stored entry, every other row unchanged).  A ring and an append cache, bf16 and fp8, one head
and four per kv head."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from hybrid_sliding_window_decode_amd import inputs
from gpu_util import CODE, assert_parity, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "layer_step")
NP_CACHE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


@pytest.mark.parametrize("kind,dtype,H,pos,S", [
    ("sliding", "bf16", 8, [600, 17, 4096], None),
    ("full", "bf16", 8, [2999, 0, 1500], 3000),
    ("sliding", "fp8", 32, [511, 3, 1000], None),
    ("full", "fp8", 32, [4000, 2047], 4001),
])
def test_layer_step_called_from_c(tmp_path, kind, dtype, H, pos, S):
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi/layer_step is not built (run the build entry point)")
    B = len(pos)
    spec = (inputs.sliding_spec(B, dtype, H=H) if kind == "sliding"
            else inputs.full_spec(B, S, dtype, H=H))
    x = inputs.make_step(spec, pos, seed=61)
    ring = kind == "sliding"
    ind, outd = tmp_path / "in", tmp_path / "out"
    ind.mkdir()
    outd.mkdir()
    for name, a in (("q", x.q), ("k", x.k), ("v", x.v), ("gate", x.gate)):
        np.ascontiguousarray(a, np.float32).tofile(ind / (name + ".bin"))
    np.ascontiguousarray(x.pos, np.int32).tofile(ind / "pos.bin")
    np.ascontiguousarray(x.k_cache).tofile(ind / "kc.bin")
    np.ascontiguousarray(x.v_cache).tofile(ind / "vc.bin")
    if spec.kv_scale is not None:
        np.ascontiguousarray(spec.kv_scale, np.float32).tofile(ind / "scale.bin")
    mp = int(x.pos.max())
    args = [EXE, str(ind), str(outd), B, spec.H, spec.Hkv, spec.D, spec.n_slots, CODE[dtype],
            int(ring), spec.rot, repr(spec.theta), mp]
    say("C-ABI layer_step %s %s H=%d pos=%s" % (kind, dtype, H, pos))
    r = subprocess.run([str(a) for a in args], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "layer_step ok" in r.stdout

    out = np.fromfile(outd / "out.bin", np.float32).reshape(B, spec.H, spec.D)
    kc = np.fromfile(outd / "kc.bin", NP_CACHE[dtype]).reshape(x.k_cache.shape)
    vc = np.fromfile(outd / "vc.bin", NP_CACHE[dtype]).reshape(x.v_cache.shape)
    kc_ref, vc_ref = x.k_cache.copy(), x.v_cache.copy()       # the oracle writes its entry here
    ref = oracle.layer_step(x.q, x.k, x.v, x.gate, kc_ref, vc_ref, x.pos, CODE[dtype], ring,
                            spec.rot, spec.theta, write=True, kv_scale=spec.kv_scale)
    assert_parity(out, ref["out"], x, "C-ABI layer_step")
    # both caches bit for bit: the entry rows as the oracle stores them,
    # every other row as it was
    bits = lambda a: np.ascontiguousarray(a).view(np.uint8)
    assert np.array_equal(bits(kc), bits(kc_ref))
    assert np.array_equal(bits(vc), bits(vc_ref))
