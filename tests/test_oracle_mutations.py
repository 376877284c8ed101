"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle (on the CPU) -- in
oracle/oracle.c, built into a library of its own, or in the Python side
(oracle/__init__.py: the acceptance check, its tolerances and the widening
of GPU results), imported in place of the real one -- and runs the pin
suite (tests/test_oracle.py) against it.  The suite must fail for every
planted mistake."""
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
    ("entries_rows_cols_swapped", "    int64_t i = rows[e], j = cols[e];", "    int64_t i = cols[e], j = rows[e];"),
    ("entries_drop_last_k", "    for (int64_t k = 0; k < K; ++k) {\n      double p = elem(a_type",
     "    for (int64_t k = 0; k + 1 < K; ++k) {\n      double p = elem(a_type"),
    ("entries_absum_signed", "      s += p;\n      t += fabs(p);\n    }\n    double r", "      s += p;\n      t += p;\n    }\n    double r"),
    ("entries_alpha_dropped", "    double r = alpha * s;\n    if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n    ref[e] = r;",
     "    double r = s;\n    if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);\n    ref[e] = r;"),
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


def run_pins_with_c_source(src):
    """Build src as the oracle library and run the pin suite against it;
    returns pytest's exit status and output."""
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
    return r.returncode, r.stdout


def test_c_side_harness_passes_the_unchanged_oracle():
    # The control: the unchanged source, built and loaded the same way,
    # passes every pin.
    st, out = run_pins_with_c_source(open(SRC).read())
    assert st == 0, out[-2000:]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(mutation):
    # (name, old, new[, old2, new2 ...]): every `old` must occur once
    name, pairs = mutation[0], list(zip(mutation[1::2], mutation[2::2]))
    src = open(SRC).read()
    for old, new in pairs:
        assert src.count(old) == 1, f"mutation {name} no longer matches oracle.c"
        src = src.replace(old, new)
    st, out = run_pins_with_c_source(src)
    # 1: tests ran and failed (not a collection or usage error)
    assert st == 1, f"the pins did not catch mutation {name} (pytest status {st}):\n{out[-2000:]}"


# (name, text in oracle/__init__.py, replacement): the Python half of the oracle.
PY_MUTATIONS = [
    ("tolerance_bf16_looser", "TOLERANCE = {BF16: (2.0 ** -8, 1e-4)", "TOLERANCE = {BF16: (2.0 ** -7, 1e-4)"),
    ("tolerance_e4m3_like_bf16", "E4M3: (2.0 ** -7, 2e-3)}", "E4M3: (2.0 ** -8, 2e-3)}"),
    ("check_ignores_alpha", "coef * abs(float(alpha)) * absum", "coef * absum"),
    ("check_lets_nan_pass", "bad = ~finite | (err > bound)", "bad = (err > bound)"),
    ("check_bound_exclusive", "bad = ~finite | (err > bound)", "bad = ~finite | (err >= bound)"),
    ("check_signed_relative_bound", "bound = rel * np.abs(ref)", "bound = rel * ref"),
    ("widen_drops_sign", "c = np.asarray(codes).view(np.uint16).astype(np.uint32) << 16",
     "c = (np.asarray(codes).view(np.uint16).astype(np.uint32) & 0x7FFF) << 16"),
    ("widen_wrong_half", "c = np.asarray(codes).view(np.uint16).astype(np.uint32) << 16",
     "c = np.asarray(codes).view(np.uint16).astype(np.uint32) << 15"),
]


def run_pins_with_python_side(src_text):
    """Run the pin suite with oracle/__init__.py replaced by src_text (in a
    temporary copy of the package, beside the original oracle.c); returns
    pytest's exit status and output."""
    import shutil
    with tempfile.TemporaryDirectory() as d:
        pkg = os.path.join(d, "oracle")
        os.makedirs(pkg)
        shutil.copy(SRC, os.path.join(pkg, "oracle.c"))
        open(os.path.join(pkg, "__init__.py"), "w").write(src_text)
        # The mutated package is imported first, so the pin suite's own
        # `import oracle` finds it in sys.modules.
        prog = ("import sys; sys.path.insert(0, %r)\n"
                "import oracle\n"
                "assert oracle.__file__.startswith(%r), oracle.__file__\n"
                "import pytest\n"
                "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', %r]))\n"
                % (d, d, os.path.join(ROOT, "tests", "test_oracle.py")))
        env = {k: v for k, v in os.environ.items() if k != "MIGEMM_ORACLE_LIB"}
        r = subprocess.run([sys.executable, "-c", prog], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=600)
    return r.returncode, r.stdout


def test_python_side_harness_passes_the_unchanged_oracle():
    # The control: the same harness on an unchanged copy passes every pin,
    # so a failure under a mutation is the mutation's doing.
    st, out = run_pins_with_python_side(open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    assert st == 0, out[-2000:]


@pytest.mark.parametrize("mutation", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_pins_catch_planted_mistake_in_python_side(mutation):
    name, old, new = mutation
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, f"mutation {name} no longer matches oracle/__init__.py"
    st, out = run_pins_with_python_side(src.replace(old, new))
    # 1: tests ran and failed (not a collection or usage error)
    assert st == 1, f"the pins did not catch mutation {name} (pytest status {st}):\n{out[-2000:]}"
