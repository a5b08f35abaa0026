"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each mutation edits a copy of oracle/focus_oracle.c the way a plausible slip
would (a dropped term, a wrong sign or index, a transposed operand, the wrong
tie rule), builds it with gcc into a temporary directory, and runs every pin
of oracle_pins.py against it.  At least one pin must fail for every mutant;
the real oracle passes all of them (test_oracle_pins.py).
"""
import os

import pytest

import oracle
from oracle import build as oracle_build

import oracle_pins as pins

MUTATIONS = [
    ("tensor scale divides by 448 only", "return amax / 2688.0f;", "return amax / 448.0f;"),
    ("block scale drops the factor 6", "float den = 6.0f * s2;", "float den = s2;"),
    ("block scale drops m", "float num = a * mb;", "float num = a;"),
    ("block scale drops the zero-block rule", "if (t == 0.0f) t = 1.0f;", ";"),
    ("block scale lower clamp 2^-9", "fmaxf(t, 0x1p-6f)", "fmaxf(t, 0x1p-9f)"),
    ("block scale upper clamp 240 (FNUZ max)", "0x1p-6f), 448.0f)", "0x1p-6f), 240.0f)"),
    ("element drops the sigmoid", "float d = (S * sig) * s2;", "float d = S * s2;"),
    ("element drops s2", "float d = (S * sig) * s2;", "float d = S * sig;"),
    ("element clamp at 4", "x = fminf(fmaxf(x, -6.0f), 6.0f);", "x = fminf(fmaxf(x, -4.0f), 4.0f);"),
    ("sigmoid uses exp(+q)", "float e = oracle_expf(-q);", "float e = oracle_expf(q);"),
    ("sigmoid drops the 1 +", "float s = 1.0f + e;", "float s = e;"),
    ("E2M1 ties to odd", "(d == best_d && (k & 1u) == 0u)", "(d == best_d && (k & 1u) == 1u)"),
    ("E2M1 ties away from zero", "(d == best_d && (k & 1u) == 0u)", "(d == best_d)"),
    ("E2M1 drops the sign", "return (sign << 3) | best;", "return best;"),
    ("E4M3 ties to odd", "(d == best_d && (b & 1u) == 0u)", "(d == best_d && (b & 1u) == 1u)"),
    ("E4M3 exponent bias 8", "ldexp(1.0 + (double)m / 8.0, (int)e - 7)",
     "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    ("BF16 truncates", "return (lo & 1u) ? hi : lo;", "return lo;"),
    ("q index swaps the sub-blocks", "q[r * (2 * nb) + 2 * b + k]", "q[r * (2 * nb) + 2 * b + 1 - k]"),
    ("q index transposed", "q[r * (2 * nb) + 2 * b + k]", "q[(2 * b + k) * rows + r]"),
    ("m index transposed", "m[r * nb + b]", "m[b * rows + r]"),
    ("nibble order swapped", "(uint8_t)(c[2 * j] | (c[2 * j + 1] << 4))",
     "(uint8_t)(c[2 * j + 1] | (c[2 * j] << 4))"),
    ("dequant drops S", "float v = (c * S) * s2;", "float v = c * s2;"),
    ("dequantize reads the wrong nibble", "(i & 1) ? (byte >> 4) : (byte & 15u)",
     "(i & 1) ? (byte & 15u) : (byte >> 4)"),
    ("s2 == 0 drops the code sign", "return ((uint32_t)w >> 15) << 3;", "return 0;"),
    ("per-token scale from the first row only", "oracle_tensor_scale(x + t * hidden, hidden, NULL)",
     "oracle_tensor_scale(x, hidden, NULL)"),
    ("FourOverSix prefers 4 on ties", "const int four = e4 < e6;", "const int four = e4 <= e6;"),
    ("FourOverSix never picks 4", "const int four = e4 < e6;", "const int four = 0;"),
    ("FourOverSix 4-candidate maps the max to 6", "fo6_candidate(wb, a, 4.0f, s2, &sb4, c4, &e4);",
     "fo6_candidate(wb, a, 6.0f, s2, &sb4, c4, &e4);"),
    ("FourOverSix error without the square", "err = err + e * e;", "err = err + fabsf(e);"),
    ("FourOverSix per-token scale from row 0", "s2_out[t] = oracle_tensor_scale(x + t * hidden, hidden, NULL);",
     "s2_out[t] = oracle_tensor_scale(x, hidden, NULL);"),
    ("MXFP4 scale rounds log2 to nearest", "int e = (e2 - 1) - 2;", "int e = (int)lrintf(log2f(t)) - 2;"),
    ("MXFP4 scale uses emax 3", "int e = (e2 - 1) - 2;", "int e = (e2 - 1) - 3;"),
    ("MXFP4 zero block gets byte 0", "if (t == 0.0f) return 127u;", "if (t == 0.0f) return 0u;"),
    ("MXFP4 ignores m", "unsigned sb = oracle_mx_block_scale(a, mb);", "unsigned sb = oracle_mx_block_scale(a, 1.0f);"),
    ("MXFP4 q indexed as NVFP4", "q[r * (4 * nb) + 4 * b + k]", "q[r * (4 * nb) + 2 * b + k]"),
    ("MXFP4 32-block max over 16", "for (int i = 0; i < 32; ++i) {\n                float v = fabsf",
     "for (int i = 0; i < 16; ++i) {\n                float v = fabsf"),
    ("E0M3 ties to odd", "if (d < best_d || (d == best_d && (k & 1u) == 0u)) {\n            best_d = d;\n            best = k;\n        }\n    }\n    return (sign << 3) | best;\n}\n\nfloat oracle_e0m3_value",
     "if (d < best_d || (d == best_d && (k & 1u) == 1u)) {\n            best_d = d;\n            best = k;\n        }\n    }\n    return (sign << 3) | best;\n}\n\nfloat oracle_e0m3_value"),
    ("E0M3 maps the block max to 6", "float t = a / (7.0f * s2);", "float t = a / (6.0f * s2);"),
    ("E0M3 clamps at 6", "x = fminf(fmaxf(x, -7.0f), 7.0f);", "x = fminf(fmaxf(x, -6.0f), 6.0f);"),
    ("MixFP4 tile index transposed", "map[(r / tile_rows) * tiles_per_row + (b * 16) / tile_cols]",
     "map[((b * 16) / tile_cols) * (rows / tile_rows) + r / tile_rows]"),
    ("MixFP4 map ignored", "int e0m3 = map[(r / tile_rows) * tiles_per_row + (b * 16) / tile_cols] != 0;",
     "int e0m3 = 0;"),
    ("MixFP4 dequantize reads every tile as E2M1",
     "float cv = e0m3 ? oracle_e0m3_value(c) : oracle_e2m1_value(c);\n                out[r * cols + b * 16 + i]",
     "float cv = oracle_e2m1_value(c);\n                out[r * cols + b * 16 + i]"),
    ("MixFP4 dequantize nibbles swapped", "unsigned c = (i & 1) ? (byte >> 4) : (byte & 15u);\n                float cv = e0m3",
     "unsigned c = (i & 1) ? (byte & 15u) : (byte >> 4);\n                float cv = e0m3"),
    ("linear drops the block scale",
     "return (double)oracle_e2m1_value(c) * (double)oracle_e4m3_value(scales[row * (K / 16) + k / 16]);",
     "return (double)oracle_e2m1_value(c);"),
    ("linear ignores the per-token s2", "double sx = (double)xs2[xs2_per_row ? t : 0];",
     "double sx = (double)xs2[0];"),
    ("linear drops the weight s2", "double s = sx * (double)ws2[0];", "double s = sx;"),
    ("linear scale of the first row only", "scales[row * (K / 16) + k / 16]", "scales[k / 16]"),
    ("linear output transposed", "y[t * N + o] = acc * s;", "y[o * M + t] = acc * s;"),
    ("linear scale per 8 elements", "scales[row * (K / 16) + k / 16]", "scales[row * (K / 16) + (k / 8) % (K / 16)]"),
    ("block max over the first sub-block only", "for (int i = 0; i < 16; ++i) {\n                float v = fabsf",
     "for (int i = 0; i < 8; ++i) {\n                float v = fabsf"),
]


def _mutant(tmp_path, old, new):
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    mutated = src.replace(old, new)
    c = os.path.join(tmp_path, "focus_oracle_mutant.c")
    with open(c, "w") as f:
        f.write(mutated)
    so = os.path.join(tmp_path, "liboracle_mutant.so")
    oracle_build.build(c, so)
    return oracle.Oracle(so)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, old, new):
    o = _mutant(str(tmp_path), old, new)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, f"planted mistake '{name}' passed every pin"
