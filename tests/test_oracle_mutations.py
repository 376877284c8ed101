"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU),
builds it, and runs the pin suite (tests/test_oracle.py) against the broken
build.  The suite must fail for every planted mistake."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement[, text, replacement ...]): one plausible
# mistake each.
MUTATIONS = [
    ("bf16_bias", "ldexp((double)(128 + f), e - 127 - 7)", "ldexp((double)(128 + f), e - 126 - 7)"),
    ("bf16_subnormal", "ldexp((double)f, 1 - 127 - 7)", "ldexp((double)f, 0 - 127 - 7)"),
    ("e4m3_subnormal", "ldexp((double)f, 1 - 7 - 3)", "ldexp((double)f, 0 - 7 - 3)"),
    ("e4m3_no_nan", "if (e == 0xF && f == 0x7) {", "if (0) {"),
    ("e4m3_bias", "ldexp((double)(8 + f), e - 7 - 3)", "ldexp((double)(8 + f), e - 8 - 3)"),
    ("drop_last_k", "for (int64_t k = 0; k < K; ++k) {\n        double p = a[k] * b[k];",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n        double p = a[k] * b[k];"),
    ("b_transposed", "Bd[j * K + k] = elem(b_type, B, b_rs, b_cs, k, j);",
     "Bd[j * K + k] = elem(b_type, B, b_rs, b_cs, j, k);"),
    ("a_strides_swapped", "Ad[i * K + k] = elem(a_type, A, a_rs, a_cs, i, k);",
     "Ad[i * K + k] = elem(a_type, A, a_cs, a_rs, i, k);"),
    ("minus_sign", "        double p = a[k] * b[k];\n        s += p;", "        double p = a[k] * b[k];\n        s -= p;"),
    ("no_abs", "        s += p;\n        t += fabs(p);", "        s += p;\n        t += p;"),
    ("beta_dropped", "      if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n      ref[i * N + j] = r;",
     "      ref[i * N + j] = r;"),
    ("alpha_on_c", "      double r = alpha * s;\n      if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n      ref[i * N + j] = r;",
     "      double r = s;\n      if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n      ref[i * N + j] = alpha * r;"),
    ("entries_c_transposed", "    if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n    ref[e] = r;",
     "    if (beta != 0.0) r += beta * elem(c_type, C, c_cs, c_rs, i, j);\n    ref[e] = r;"),
    ("rowsum_in_double", "volatile float s = 0.0f;", "volatile double s = 0.0;"),
    ("rowsum_from_minus_zero", "volatile float s = 0.0f;", "volatile float s = -0.0f;"),
    ("rowsum_descending", "      for (int64_t j = j0; j < j1; ++j) {\n        float v",
     "      for (int64_t j = j1 - 1; j >= j0; --j) {\n        float v"),
    ("rowsum_two_partials",
     "        s = s + v;\n        if (!isnan(v)) m = max_signed_zero(m, v);\n      }\n      row_sum[r * ld + t] = s;",
     "        if (((j - j0) & 1) == 0) s = s + v; else s2 = s2 + v;\n"
     "        if (!isnan(v)) m = max_signed_zero(m, v);\n      }\n      row_sum[r * ld + t] = s + s2;",
     "      float m = -INFINITY;\n", "      float m = -INFINITY;\n      volatile float s2 = 0.0f;\n"),
    ("rowsum_skips_last_column", "      for (int64_t j = j0; j < j1; ++j) {\n        float v",
     "      for (int64_t j = j0; j + 1 < j1; ++j) {\n        float v"),
    ("rowmax_from_zero", "float m = -INFINITY;", "float m = 0.0f;"),
    ("max_signed_zero_ignored", "return signbit(a) ? b : a;", "return a;"),
    ("max_keeps_nan", "if (!isnan(v)) m = max_signed_zero(m, v);", "m = max_signed_zero(m, v);"),
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(mutation):
    # (name, old, new[, old2, new2 ...]): every `old` must occur once
    name, pairs = mutation[0], list(zip(mutation[1::2], mutation[2::2]))
    src = open(SRC).read()
    for old, new in pairs:
        assert src.count(old) == 1, f"mutation {name} no longer matches oracle.c"
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        msrc = os.path.join(d, "oracle_mut.c")
        lib = os.path.join(d, "liboracle_mut.so")
        open(msrc, "w").write(src)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
                        "-o", lib, msrc, "-lm"], check=True)
        env = dict(os.environ, MIGEMM_ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"the pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
