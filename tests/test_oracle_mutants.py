"""Each pin set must reject plausible mistakes in the oracle (CPU only).

A mutant is a copy of the oracle's C source with one planted mistake (a
dropped term, a wrong sign, index or constant, a reordered step), compiled
into its own library.  Every mutant must fail at least one pin; a mutant that
passes them all would mean the pins cannot tell that mistake apart.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

# (name, [(text in the oracle source, replacement), ...])
MUTANTS = [
    ("ring slot off by one", [("int row = ring ? p % n_slots : p;",
                               "int row = ring ? (p + 1) % n_slots : p;")]),
    ("window one key too wide", [("int n = p < n_slots ? p : n_slots;",
                                  "int n = p + 1 < n_slots ? p + 1 : n_slots;")]),
    ("write before read", [
        ("    if (write) status = orc_write_entry(B, Hkv, D, n_slots, dtype, ring, pos, kh, vh, k_cache, v_cache);\n", ""),
        ("    int status = 0;\n",
         "    int status = 0;\n    if (write) status = orc_write_entry(B, Hkv, D, n_slots, dtype, ring, pos, kh, vh, k_cache, v_cache);\n")]),
    ("mask one slot too many", [("mask[(size_t)b * n_slots + s] = (uint8_t)(s < n_valid);",
                                 "mask[(size_t)b * n_slots + s] = (uint8_t)(s <= n_valid);")]),
    ("rope pairs adjacent instead of rotate-half", [
        ("int i0 = interleaved ? 2 * i : i;", "int i0 = interleaved ? i : 2 * i;"),
        ("int i1 = interleaved ? 2 * i + 1 : i + half;", "int i1 = interleaved ? i + half : 2 * i + 1;")]),
    ("rope exponent over head_dim", [("pow(theta, -2.0 * (double)i / (double)rot)",
                                      "pow(theta, -2.0 * (double)i / (double)D)")]),
    ("rope sign of sine", [("out[i0] = x0 * c - x1 * s;", "out[i0] = x0 * c + x1 * s;")]),
    ("rope at pos + 1", [("(int64_t)pos[v / per_pos], interleaved);",
                          "(int64_t)pos[v / per_pos] + 1, interleaved);")]),
    ("new entry missing from the normaliser", [("    double l = w_new;\n", "    double l = 0.0 * w_new;\n")]),
    ("new entry value dropped", [("for (int d = 0; d < D; ++d) o[d] = w_new * v_new[d];",
                                  "for (int d = 0; d < D; ++d) o[d] = 0.0 * v_new[d];")]),
    ("score scale dropped", [("        s[j] = scale * acc;\n        if (s[j] > m) m = s[j];",
                              "        s[j] = acc;\n        if (s[j] > m) m = s[j];")]),
    ("new key left unrounded", [("    orc_decode(dtype, kh, nkv, khd);\n",
                                 "    for (size_t i = 0; i < nkv; ++i) khd[i] = kr[i];\n")]),
    ("merge without rescale", [("        double w = exp(m[i] - M);\n        L += l[i] * w;",
                                "        double w = 1.0 + 0.0 * exp(m[i] - M);\n        L += l[i] * w;")]),
    ("partial normaliser from the wrong max", [("        double w = exp(s[j - j0] - m);",
                                               "        double w = exp(s[j - j0]);")]),
    ("kv head mapping modulo", [("int b = bh / H, h = bh % H, g = h / G;",
                                 "int b = bh / H, h = bh % H, g = h % Hkv;")]),
    ("gate sign", [("return 1.0 / (1.0 + exp(-g));", "return 1.0 / (1.0 + exp(g));")]),
    ("rounding truncates", [("return rint(ax / quantum) * quantum;",
                             "return floor(ax / quantum) * quantum;")]),
    ("ties away from zero", [("return rint(ax / quantum) * quantum;",
                              "return round(ax / quantum) * quantum;")]),
    ("f16 overflow threshold", [("if (ax >= 65520.0)", "if (ax > 65504.0)")]),
    ("f16 subnormal exponent", [("round_to_grid(ax, 10, -14);", "round_to_grid(ax, 10, -15);")]),
    ("f16 decode subnormal scale", [("else if (e == 0) v = ldexp((double)m, -24);",
                                     "else if (e == 0) v = ldexp((double)m, -25);")]),
    ("gate weight transposed", [("(double)w[(size_t)h * hidden + i];", "(double)w[(size_t)i * H + h];")]),
    ("fp8 without saturation", [("    if (r > 448.0) r = 448.0;\n", "")]),
    ("fp8 decode exponent bias", [("else v = ldexp((double)(8 + m), e - 10);",
                                   "else v = ldexp((double)(8 + m), e - 9);")]),
    ("V scale dropped", [("o[d] += w * (vs * load_elt(vc, dtype, (size_t)j * D + d));",
                          "o[d] += w * (1.0 * load_elt(vc, dtype, (size_t)j * D + d));")]),
    ("K scale dropped", [("acc += q[d] * (ks * load_elt(kc, dtype, (size_t)j * D + d));\n        s[j] = scale * acc;",
                          "acc += q[d] * (1.0 * load_elt(kc, dtype, (size_t)j * D + d));\n        s[j] = scale * acc;")]),
    ("entry stored unscaled", [("        kq[i] = (float)((double)kr32[i] / ks);",
                                "        kq[i] = (float)((double)kr32[i] / 1.0);")]),
    ("append capacity off by one", [("if (!ring && p >= n_slots) { status = -4; continue; }",
                                     "if (!ring && p > n_slots) { status = -4; continue; }")]),
    # the per-(stream, head) entry of the full-size checks
    ("block entry key unscaled", [("for (int d = 0; d < D; ++d) { kn[d] *= ks; vn[d] *= vs; }",
                                   "for (int d = 0; d < D; ++d) { vn[d] *= vs; }")]),
    ("block entry value scaled twice", [("for (int d = 0; d < D; ++d) { kn[d] *= ks; vn[d] *= vs; }",
                                         "for (int d = 0; d < D; ++d) { kn[d] *= ks; vn[d] *= vs * vs; }")]),
    ("block entry decoded as the wrong type", [
        ("    orc_decode(dtype, k_hat, (size_t)D, kn);",
         "    orc_decode(dtype == ORC_BF16 ? ORC_F16 : dtype, k_hat, (size_t)D, kn);")]),
]


def _apply(src, subs):
    for old, new in subs:
        assert src.count(old) == 1, "mutant anchor not unique or missing: %r" % old
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name,subs", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(tmp_path, name, subs):
    src = _apply(open(obuild.SRC).read(), subs)
    path = os.path.join(str(tmp_path), "mut.c")
    with open(path, "w") as f:
        f.write(src)
    lib = obuild.build(path, os.path.join(str(tmp_path), "libmut.so"))
    L = oracle.lib(lib)
    caught = []
    for pin in pins.QUICK_PINS:
        try:
            pin(L)
        except (AssertionError, ValueError, FloatingPointError, ZeroDivisionError) as e:
            caught.append((pin.__name__, repr(e)[:80]))
    assert caught, "mutant '%s' passed every pin" % name
