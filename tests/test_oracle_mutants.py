"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake in a copy of ``oracle/oracle.c`` (on the CPU, in
a temporary directory), builds it, and runs the pin suite against that build
in a subprocess; the suite must fail.  The unmodified source must pass.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "transposed_weight": ("(double)w[k]", "(double)W[k * N + n]"),
    "dropped_bias": ("Y[r * N + n] = acc + (double)b[n];", "Y[r * N + n] = acc;"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "wrong_row": ("const float *x = X + rows[r] * K;", "const float *x = X + r * K;"),
    "tanh_gelu": ("return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
                  "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "clamp_before_scale": ("double t = y[i] * s;\n        t = hardtanh(t, lo, hi);",
                           "double t = hardtanh(y[i], lo, hi) * s;"),
    "pool_divisor": ("out[r * L + j] = acc / (double)k;", "out[r * L + j] = acc / (double)(k + 1);"),
    "pool_ceil_mode": ("int64_t L = (N - k) / st + 1;", "int64_t L = (N + st - 1) / st;"),
    "scale_before_gelu": ("double v = gelu_erf(pooled[r * L + j]) * s;", "double v = gelu_erf(pooled[r * L + j] * s);"),
    "max_of_pooled_then_gelu": ("double v = gelu_erf(pooled[r * L + j]) * s;", "double v = pooled[r * L + j] * s;"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-y));", "return 1.0 / (1.0 + exp(y));"),
    "swish_scale_dropped": ("out[i] = (y[i] * sigmoid(y[i])) * s;", "out[i] = y[i] * sigmoid(y[i]);"),
}


def _build(tmp_path, text, name):
    src = tmp_path / (name + ".c")
    src.write_text(text)
    lib = tmp_path / ("lib" + name + ".so")
    subprocess.run(["gcc", *oracle._CFLAGS, str(src), "-o", str(lib), "-lm"], check=True)
    return str(lib)


def _run_pins(lib):
    env = dict(os.environ, LIN_EPI_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_oracle_passes(tmp_path):
    with open(SRC) as f:
        text = f.read()
    rc, out = _run_pins(_build(tmp_path, text, "clean"))
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation site not found: %s" % name
    rc, out = _run_pins(_build(tmp_path, text.replace(old, new), name))
    assert rc != 0, "pins accepted the planted mistake %s:\n%s" % (name, out)
