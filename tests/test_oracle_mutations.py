"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/moe_oracle.c, plants one plausible mistake (a dropped
term, a wrong index or rounding, a reversed order, a wrong constant), builds
the copy with gcc into a temporary directory and runs tests/test_oracle.py
against it in a child process.  The pins must fail for every one.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "moe_oracle.c")

MUTATIONS = [
    ("combine adds a stray term", "acc[h] = have ? acc[h] + v : v;",
     "acc[h] = have ? acc[h] + v : v + 0.0f * acc[h] + (h == 0 ? 1.0f : 0.0f);"),
    ("combine drops the last slot", "for (int32_t j = 0; j < k; ++j) {\n            if (!primary_local",
     "for (int32_t j = 0; j < k - (k > 2); ++j) {\n            if (!primary_local"),
    ("padding rounds up one too far", "int32_t padded = ((tpe[e] + P - 1) / P) * P;",
     "int32_t padded = ((tpe[e] + P) / P) * P;"),
    ("rows in descending token order", "for (int64_t t = 0; t < T; ++t) {\n            if (!map[t * E + lb + e])",
     "for (int64_t t = T - 1; t >= 0; --t) {\n            if (!map[t * E + lb + e])"),
    ("repeated ids not merged", "W[t * E + e] = W[t * E + e] + w[t * k + j];", "W[t * E + e] = w[t * k + j];"),
    ("ties round away from even", "return (lo & 1u) ? hi : lo;", "return hi;"),
    ("dw products rounded to fp32",
     "s += bf16_value(grad_out[t * H + h]) * bf16_value(F[r * H + h]);",
     "s += (float)(bf16_value(grad_out[t * H + h]) * bf16_value(F[r * H + h]));"),
    ("sentinel expert id wrong", "row_expert[r] = EL;", "row_expert[r] = -1;"),
    ("no repeated-id check in combine", "for (int32_t q = 0; q < j; ++q)", "for (int32_t q = 0; q < 0; ++q)"),
    ("slot mapped to the next expert's row", "if (idx[t * k + j] == (int64_t)lb + e)",
     "if (idx[t * k + j] == (int64_t)lb + e + 1)"),
    ("counts read one expert over", "c += map[t * E + lb + e];", "c += map[t * E + lb + (e + 1) % EL];"),
    ("weight gradient of repeated ids dropped",
     "grad_topk_w[t * k + j] = (local && r >= 0 && r < R && grad_row_w) ? grad_row_w[r] : 0.0f;",
     "grad_topk_w[t * k + j] = (local && r >= 0 && r < R && grad_row_w && (j == 0 || idx[t * k + j - 1] != e)) ? grad_row_w[r] : 0.0f;"),
    ("pad rows keep data", "row_w[r] = 0.0f;\n            if (rows)\n                memset(rows + r * H, 0,",
     "row_w[r] = 0.0f;\n            if (rows)\n                memset(rows + r * H, 1,"),
    ("sentinel rows keep data",
     "memset(rows + r * H, 0, (size_t)H * sizeof(uint16_t));\n    }\n\n    free(W);",
     "memset(rows + r * H, 1, (size_t)H * sizeof(uint16_t));\n    }\n\n    free(W);"),
    ("sentinel rows left unwritten",
     "memset(rows + r * H, 0, (size_t)H * sizeof(uint16_t));\n    }\n\n    free(W);",
     "(void)0;\n    }\n\n    free(W);"),
    ("combine leaves tokens without a local slot unwritten",
     "for (int64_t h = 0; h < H; ++h) {\n            float s = have ? acc[h] : 0.0f;",
     "for (int64_t h = 0; h < H * have; ++h) {\n            float s = have ? acc[h] : 0.0f;"),
    ("local range starts one expert late", "if (e < 0 || e >= E || e < lb || e >= (int64_t)lb + EL)",
     "if (e < 0 || e >= E || e <= lb || e >= (int64_t)lb + EL)"),
    ("probs written as the plain multihot", "probs[i] = map[i] ? W[i] : 0.0f;",
     "probs[i] = map[i] ? 1.0f : 0.0f;"),
]

# FP8 dispatch, caught by tests/test_oracle_fp8.py
FP8_MUTATIONS = [
    ("e4m3 ties to the odd code", "(dc == db && (c & 1) == 0 && (best & 1) != 0)",
     "(dc == db && (c & 1) != 0)"),
    ("e4m3 subnormal step halved", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("amax over half the block", "for (int i = 0; i < 128; ++i) {\n            float m",
     "for (int i = 0; i < 64; ++i) {\n            float m"),
    ("no floor under amax", "float a = amax > 1e-4f ? amax : 1e-4f;", "float a = amax;"),
    ("scale inverted", "float s = a / 448.0f;", "float s = 448.0f / a;"),
    ("pad rows get a nonzero scale", "row_scale[r * nb + b] = 0.0f;", "row_scale[r * nb + b] = 1.0f;"),
]


CASES = ([m + ("test_oracle.py",) for m in MUTATIONS]
         + [m + ("test_oracle_fp8.py",) for m in FP8_MUTATIONS])


@pytest.mark.parametrize("label,old,new,pins", CASES, ids=[m[0] for m in CASES])
def test_planted_mistake_is_caught(label, old, new, pins, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {label}"
    mutated = tmp_path / "moe_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "liboracle_mut.so"))
    env = dict(os.environ, MOE_ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, pins),
                          "-x", "-q", "-p", "no:cacheprovider"],
                         env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"the pins did not catch: {label}\n{res.stdout[-2000:]}"
