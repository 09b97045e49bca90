"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutation below is a plausible slip in coli_oracle.c (a dropped term, a
wrong sign, index or rounding mode, a transposed operand).  The mutant is
compiled into a temporary library and every pin of tests/oracle_pins.py is
run against it; the test passes only if some pin rejects the mutant.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "coli_oracle.c")

MUTANTS = {
    "q8 rounds half away from zero": ("v = lrintf(xb[j] / db);", "v = lroundf(xb[j] / db);"),
    "q4 rounds half away from zero": ("v = lrintf(w[j] / sc);", "v = lroundf(w[j] / sc);"),
    "q8 scale over 128": ("const float db = amax / 127.0f;", "const float db = amax / 128.0f;"),
    "q4 scale over 8": ("const float sc = amax / 7.0f;", "const float sc = amax / 8.0f;"),
    "q8 quotient by reciprocal": ("v = lrintf(xb[j] / db);", "v = lrintf(xb[j] * (1.0f / db));"),
    "unpack sign threshold": ("q[2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);",
                              "q[2 * i] = (int8_t)(lo > 8 ? lo - 16 : lo);"),
    "pack nibble order swapped":
        ("out[i] = (uint8_t)(((uint8_t)q[2 * i] & 0x0F) | (((uint8_t)q[2 * i + 1] & 0x0F) << 4));",
         "out[i] = (uint8_t)(((uint8_t)q[2 * i + 1] & 0x0F) | (((uint8_t)q[2 * i] & 0x0F) << 4));"),
    "partials even/odd columns swapped":
        ("acc += w0 * (int32_t)xq[32 * b + 2 * j] + w1 * (int32_t)xq[32 * b + 2 * j + 1];",
         "acc += w1 * (int32_t)xq[32 * b + 2 * j] + w0 * (int32_t)xq[32 * b + 2 * j + 1];"),
    "partials high nibble unsigned":
        ("const int w0 = lo >= 8 ? lo - 16 : lo, w1 = hi >= 8 ? hi - 16 : hi;",
         "const int w0 = lo >= 8 ? lo - 16 : lo, w1 = hi;"),
    "rescale drops the row scale": ("return acc * s;\n}", "return acc;\n}"),
    "rescale uses the next block's scale":
        ("for (int64_t b = 0; b < nb; ++b) acc = fmaf((float)P[b], d[b], acc);",
         "for (int64_t b = 0; b < nb; ++b) acc = fmaf((float)P[b], d[(b + 1) % nb], acc);"),
    "exp drops the 1/4! term": ("p = fmaf(p, r, 4.16666666666666667e-02f);", ""),
    "exp ln2 low part sign": ("r = fmaf(-n, 1.42860676533018708e-06f, r);",
                              "r = fmaf(n, 1.42860676533018708e-06f, r);"),
    "sigmoid sign": ("float orc_sigmoidf(float x) { return 1.0f / (1.0f + orc_expf(-x)); }",
                     "float orc_sigmoidf(float x) { return 1.0f / (1.0f + orc_expf(x)); }"),
    "silu sign": ("float orc_siluf(float g) { return g / (1.0f + orc_expf(-g)); }",
                  "float orc_siluf(float g) { return g / (1.0f + orc_expf(g)); }"),
    "route tie goes to the higher index": ("if (best < 0 || c[e] > c[best]) best = e;",
                                           "if (best < 0 || c[e] >= c[best]) best = e;"),
    "route selects without the bias": ("c[e] = s[e] + bias[e];", "c[e] = s[e];"),
    "route weights include the bias":
        ("w[t * k + j] = (s[idx[t * k + j]] / sum) * routed_scale;",
         "w[t * k + j] = (c[idx[t * k + j]] / sum) * routed_scale;"),
    "route ignores routed_scale": ("(s[idx[t * k + j]] / sum) * routed_scale;",
                                   "(s[idx[t * k + j]] / sum);"),
    "swiglu uses the gate twice": ("h[r] = orc_siluf(g[r]) * u[r];", "h[r] = orc_siluf(g[r]) * g[r];"),
    "down projection skips Q8(h) scale":
        ("orc_matvec(down_q, bits, down_s, D, F, hq, hd, o, P_down, abs_down);",
         "orc_matvec(down_q, bits, gate_s, D, F, hq, hd, o, P_down, abs_down);"),
    "int8 weights scale over 128": ("const float sw = amax / 127.0f;",
                                    "const float sw = amax / 128.0f;"),
    "int8 weights round half away from zero": ("v = lrintf(w[j] / sw);", "v = lroundf(w[j] / sw);"),
    "int8 weights clamp at 63": ("    if (v > 127) v = 127;\n    if (v < -127) v = -127;\n    q[j]",
                                 "    if (v > 63) v = 63;\n    if (v < -127) v = -127;\n    q[j]"),
    "int8 partials read unsigned codes":
        ("const int8_t* w8 = (const int8_t*)wrow + 32 * b;", "const uint8_t* w8 = wrow + 32 * b;"),
    "int8 rows at the nibble stride": ("Wq + r * (k * bits / 8)", "Wq + r * (k / 2)"),
    "int2 ties away from zero": ("if (s2 != 0.0f) v = lrintf(w[j] / s2);",
                                 "if (s2 != 0.0f) v = lroundf(w[j] / s2);"),
    "int2 scale over 2": ("const float s2 = amax / 1.0f;", "const float s2 = amax / 2.0f;"),
    "int2 decode sign threshold": ("q[4 * i + j] = (int8_t)(f >= 2 ? f - 4 : f);",
                                   "q[4 * i + j] = (int8_t)(f > 2 ? f - 4 : f);"),
    "int2 dot reads fields unsigned": ("acc += (f >= 2 ? f - 4 : f) * (int32_t)xq[32 * b + j];",
                                       "acc += f * (int32_t)xq[32 * b + j];"),
    "int2 field order reversed": ("byte |= (uint8_t)(((uint8_t)q[4 * i + j] & 3u) << (2 * j));",
                                  "byte |= (uint8_t)(((uint8_t)q[4 * i + j] & 3u) << (2 * (3 - j)));"),
    "tier evicts the most recently used": ("if (v < 0 || stamp[s] < stamp[v]) v = s;",
                                           "if (v < 0 || stamp[s] > stamp[v]) v = s;"),
    "tier evicts pinned slots": ("if (pinned[s] || stamp[s] >= step) continue;",
                                 "if (stamp[s] >= step) continue;"),
    "tier fit check counts hit slots as free": ("if (miss > unpinned - hit_unpinned) rc = -1;",
                                                "if (miss > unpinned) rc = -1;"),
    "tier hits leave the stamp": ("    stamp[slot_of[e]] = step;\n    ++nh;", "    ++nh;"),
    "tier usage skips the shared expert": ("  if (S) count[E] = (int32_t)T;", ""),
    "pin ranking ties to the higher id": ("if (best < 0 || usage[e] > usage[best]) best = e;",
                                          "if (best < 0 || usage[e] >= usage[best]) best = e;"),
    "combine drops the shared expert": ("for (int64_t r = 0; r < D; ++r) { y[r] = o[r]; my[r] = m[r]; }",
                                        "for (int64_t r = 0; r < D; ++r) { y[r] = 0.0f; my[r] = m[r]; }"),
    "combine ignores routing weights": ("y[r] = fmaf(wj, o[r], y[r]);", "y[r] = y[r] + o[r];"),
    "residual not added": ("out[t * D + r] = accumulate ? out[t * D + r] + y[r] : y[r];",
                           "out[t * D + r] = y[r];"),
    "rmsnorm divides by D-1": ("sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)(D - 1) + (double)eps)"),
    "rmsnorm drops eps": ("sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)D)"),
    "dispatch shared slot 0": ("lists[(int64_t)e * T + counts[e]++] = (int32_t)(t * (k + S) + k);",
                               "lists[(int64_t)e * T + counts[e]++] = (int32_t)(t * (k + S));"),
    "dispatch accepts repeats": ("if (idx[t * k + i] == idx[t * k + j]) return -1;",
                                 "if (0) return -1;"),
    "keep ignores repeats": ("        if (idx[t * k + i] == e) ok = 0;", "        if (0) ok = 0;"),
    "keep compares with later slots": ("      for (int32_t i = 0; i < j; ++i)\n        if (idx[t * k + i] == e) ok = 0;",
                                       "      for (int32_t i = j + 1; i < k; ++i)\n        if (idx[t * k + i] == e) ok = 0;"),
    "keep accepts index E": ("      int ok = e >= 0 && e < E;", "      int ok = e >= 0 && e <= E;"),
    "layer ignores keep": ("      if (j >= 0 && keep && !keep[t * k + j]) continue;", ""),
    "dispatch lists dropped entries": ("        if (idx[t * k + j] == e && (!keep || keep[t * k + j]))",
                                       "        if (idx[t * k + j] == e)"),
    "router logits summed in fp32":
        ("    double s = 0.0;\n    for (int64_t d = 0; d < D; ++d) s += (double)wr[e * D + d] * (double)x[t * D + d];",
         "    float s = 0.0f;\n    for (int64_t d = 0; d < D; ++d) s += wr[e * D + d] * x[t * D + d];"),
    "router weights transposed":
        ("s += (double)wr[e * D + d] * (double)x[t * D + d];",
         "s += (double)wr[d * E + e] * (double)x[t * D + d];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", "-I", os.path.join(ROOT, "oracle"), str(mutant), "-o", str(lib),
                    "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant '{name}'"
