"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake in a copy of the oracle (``oracle/oracle.c`` or
the dispatch layer ``oracle/__init__.py`` that every GPU parity test goes
through), on the CPU, in a temporary copy of the package next to copies of
the pin suite and its fixtures, and runs the pin suite there in a
subprocess; the suite must fail.  The unmodified copy must pass.
"""

import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")

# name -> (file, text to replace, replacement)
MUTANTS = {
    # the arithmetic (oracle.c)
    "transposed_weight": ("c", "(double)w[k]", "(double)W[k * N + n]"),
    "dropped_bias": ("c", "Y[r * N + n] = acc + (double)b[n];", "Y[r * N + n] = acc;"),
    "dropped_last_term": ("c", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "wrong_row": ("c", "const float *x = X + rows[r] * K;", "const float *x = X + r * K;"),
    "tanh_gelu": ("c", "return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
                  "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "clamp_before_scale": ("c", "double t = y[i] * s;\n        t = hardtanh(t, lo, hi);",
                           "double t = hardtanh(y[i], lo, hi) * s;"),
    "pool_divisor": ("c", "out[r * L + j] = acc / (double)k;", "out[r * L + j] = acc / (double)(k + 1);"),
    "pool_ceil_mode": ("c", "int64_t L = (N - k) / st + 1;", "int64_t L = (N + st - 1) / st;"),
    "scale_before_gelu": ("c", "double v = gelu_erf(pooled[r * L + j]) * s;",
                          "double v = gelu_erf(pooled[r * L + j] * s);"),
    "max_of_pooled_then_gelu": ("c", "double v = gelu_erf(pooled[r * L + j]) * s;",
                                "double v = pooled[r * L + j] * s;"),
    "sigmoid_sign": ("c", "return 1.0 / (1.0 + exp(-y));", "return 1.0 / (1.0 + exp(y));"),
    "swish_scale_dropped": ("c", "out[i] = (y[i] * sigmoid(y[i])) * s;", "out[i] = y[i] * sigmoid(y[i]);"),
    # the dispatch (apply_tail / forward_rows)
    "kind1_lo_hi_swapped": ("py", "return tail_scale_hardtanh_gelu(y, scale, lo, hi)",
                            "return tail_scale_hardtanh_gelu(y, scale, hi, lo)"),
    "kind1_scale_dropped": ("py", "return tail_scale_hardtanh_gelu(y, scale, lo, hi)",
                            "return tail_scale_hardtanh_gelu(y, 1.0, lo, hi)"),
    "kind2_window_fixed_at_16": ("py", "return tail_pool_gelu_scale_rowmax(y, pool_kernel, scale)[0]",
                                 "return tail_pool_gelu_scale_rowmax(y, 16, scale)[0]"),
    "kind3_scale_dropped": ("py", "return tail_swish_scale(y, scale)", "return tail_swish_scale(y, 1.0)"),
    "kind4_pooled_by_window": ("py", "return tail_pool_gelu_scale_rowmax(y, 1, scale)[0]",
                               "return tail_pool_gelu_scale_rowmax(y, pool_kernel, scale)[0]"),
    "kind4_scale_dropped": ("py", "return tail_pool_gelu_scale_rowmax(y, 1, scale)[0]",
                            "return tail_pool_gelu_scale_rowmax(y, 1, 1.0)[0]"),
    "forward_rows_ignores_rows": ("py", "return apply_tail(linear_rows(X, W, b, rows), kind, **tail)",
                                  "return apply_tail(linear_rows(X, W, b), kind, **tail)"),
}


def _tree(tmp_path, c_text, py_text):
    """A copy of the oracle package, the input generator and the pin suite
    (with its fixtures) under tmp_path; returns (root, path of liboracle)."""
    root = tmp_path / "tree"
    (root / "oracle").mkdir(parents=True)
    (root / "oracle" / "oracle.c").write_text(c_text)
    (root / "oracle" / "__init__.py").write_text(py_text)
    shutil.copy(os.path.join(ROOT, "workloads.py"), root / "workloads.py")
    shutil.copy(os.path.join(ROOT, "pytest.ini"), root / "pytest.ini")
    (root / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), root / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), root / "tests" / "golden")
    lib = root / "oracle" / "liboracle.so"
    subprocess.run(["gcc", *oracle._CFLAGS, str(root / "oracle" / "oracle.c"), "-o", str(lib), "-lm"], check=True)
    return root, str(lib)


def _run_pins(root, lib):
    env = dict(os.environ, LIN_EPI_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        str(root / "tests" / "test_oracle_pins.py")],
                       cwd=str(root), env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def _sources():
    with open(C_SRC) as f:
        c_text = f.read()
    with open(PY_SRC) as f:
        py_text = f.read()
    return c_text, py_text


def test_unmodified_oracle_passes(tmp_path):
    rc, out = _run_pins(*_tree(tmp_path, *_sources()))
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    which, old, new = MUTANTS[name]
    c_text, py_text = _sources()
    text = c_text if which == "c" else py_text
    assert text.count(old) == 1, "mutation site not found: %s" % name
    text = text.replace(old, new)
    if which == "c":
        c_text = text
    else:
        py_text = text
    root, lib = _tree(tmp_path, c_text, py_text)
    # the copy, not the repository's package, is what the pins import
    rc, out = _run_pins(root, lib)
    assert rc != 0, "pins accepted the planted mistake %s:\n%s" % (name, out)
