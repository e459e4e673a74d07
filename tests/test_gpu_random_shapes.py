"""GPU parity over fixed, seeded draws of layer shapes: cache type, head
dim, query heads per kv head (every kernel and piece route: 1, 2, 3, 4, 5,
8, 16 in the first draw; 2, 3, 6, 7, 8, 12 in the second, mostly groups
that leave heads idle; fp8 groups of 2 in a third), streams, capacity, chunk size (library default or a
multiple of the quantum) and ragged positions from 0 to the capacity, each
a fused layer step against the oracle, the same bits as the separate
entries, and the stored entry (the checks of
test_gpu_gqa.check_layer_step).  The draws are fixed, so each case is
reproducible by its id."""
import numpy as np
import pytest

from test_gpu_gqa import check_layer_step

pytestmark = pytest.mark.gpu

ELT = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def draw(n, seed=2024, groups=(1, 2, 3, 4, 5, 8, 16)):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        kind = ["sliding", "full"][rng.integers(2)]
        dtype = ["f32", "f16", "bf16", "fp8"][rng.integers(4)]
        G = int(groups[rng.integers(len(groups))])
        D = int([64, 128, 256][rng.integers(3)])
        if dtype == "f32" and G > 1:
            continue                      # grouped f32 caches are refused
        if D == 64 and (G > 1 or dtype == "fp8"):
            continue                      # so are grouped and fp8 layers at 64 dims
        B = int(rng.integers(1, 7))
        S = None if kind == "sliding" else int(rng.integers(300, 9001))
        quantum = 32768 // (D * ELT[dtype])
        kps = int([0, 0, quantum, 2 * quantum, 4 * quantum][rng.integers(5)])
        Hkv = int([1, 2, 8][rng.integers(3)]) if G < 8 else int(rng.integers(1, 3))
        cases.append((kind, dtype, G, D, B, "ragged", S, kps, G * Hkv))
    return cases


CASES = (draw(24) + draw(16, seed=7, groups=(2, 3, 6, 7, 8, 12))
         + [c for c in draw(40, seed=11, groups=(2,)) if c[1] == "fp8"][:4])


@pytest.mark.parametrize("kind,dtype,G,D,B,pos,S,kps,H", CASES,
                         ids=["%s-%s-G%d-D%d-B%d-S%s-k%d-H%d" % (c[0], c[1], c[2], c[3], c[4], c[6],
                                                              c[7], c[8]) for c in CASES])
def test_random_shape(kind, dtype, G, D, B, pos, S, kps, H):
    check_layer_step(kind, dtype, G, D, B, pos, S, kps, H=H)
