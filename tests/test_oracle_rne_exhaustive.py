"""The oracle's float32 -> float16 / bfloat16 rounding against numpy's
float16 cast and torch's bfloat16 cast (both IEEE round to nearest, ties to
even).  CPU only.

By default every 64th float32 bit pattern is checked (2^26 inputs, a few
seconds) on top of the tie/edge set the quick pin covers; with
HSWD_EXHAUSTIVE=1 all 2^32 patterns are checked (about ten minutes)."""
import os

import numpy as np

import oracle
import pins


def test_rne_float32_sweep():
    L = oracle.lib()
    full = os.environ.get("HSWD_EXHAUSTIVE") == "1"
    stride = 1 if full else 64
    chunk = 1 << 25
    for start in range(0, 1 << 32, chunk * stride):
        u = (np.arange(chunk, dtype=np.uint64) * stride + start).astype(np.uint32)
        pins.check_rne(L, u.view(np.float32))
