"""CPU oracle for the fused fp32 linear layer + elementwise tail.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and the two share no code: this side is ``oracle.c`` (binary64,
naive loops, OpenMP over output columns) plus the thin ctypes marshalling
below.

What it computes, in the pages' order and unfused:

* ``y = x @ W^T + b`` -- nn.Linear with W of shape [out, in]
  (page "Kimi-K2.6 l2_p98", step 1 of its reading of the reference model;
  page "Kimi-K2.6 l2_p59", problem analysis).
* tail (a) ``GELU(hardtanh(y * s, lo, hi))`` -- page "Kimi-K2.6 l2_p53",
  problem statement (GEMM, scale, Hardtanh clamp, GELU).
* tail (b) ``max_j s * GELU(AvgPool1d_k(y)[j])`` -- page "Kimi-K2.6 l2_p98",
  steps 2-5 (AvgPool1d with stride = kernel, no padding, floor mode; GELU;
  scale; max over dim 1).
* tail (c) ``(y * sigmoid(y)) * s`` -- page "Kimi-K2.6 l2_p59", problem
  analysis (swish, then scaling).

Every function here is pinned by ``tests/test_oracle_pins.py`` against brute
force, closed forms, invariants and the worked example of page l2_p98,
including the dispatch ``apply_tail``/``forward_rows`` for every kind (kind 4
by page l2_p98's fold identity: it must equal tail (b) of the unpooled layer),
and ``tests/test_oracle_mutants.py`` checks that the pins reject mistakes
planted in ``oracle.c`` and in this file.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

# Test hook: a path to an alternative build of oracle.c (used only by the
# mutation test that checks the pins reject deliberately broken oracles).
_ENV_LIB = "LIN_EPI_ORACLE_LIB"


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(_ENV_LIB) or build()
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        d = ctypes.c_double
        lib.oracle_linear_rows.argtypes = [i64, i64, i64, p, p, p, p, i64, p]
        lib.oracle_linear_rows.restype = None
        lib.oracle_gelu.argtypes = [p, i64, p]
        lib.oracle_gelu.restype = None
        lib.oracle_tail_scale_hardtanh_gelu.argtypes = [p, i64, d, d, d, p]
        lib.oracle_tail_scale_hardtanh_gelu.restype = None
        lib.oracle_avgpool1d.argtypes = [p, i64, i64, i64, i64, p]
        lib.oracle_avgpool1d.restype = i64
        lib.oracle_tail_gelu_scale_rowmax.argtypes = [p, i64, i64, d, p, p]
        lib.oracle_tail_gelu_scale_rowmax.restype = None
        lib.oracle_tail_swish_scale.argtypes = [p, i64, d, p]
        lib.oracle_tail_swish_scale.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs X, W, b must be float32, got %s" % a.dtype)
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    """OpenMP threads the linear layer runs on (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def linear_rows(X, W, b, rows=None) -> np.ndarray:
    """y[r, n] = b[n] + sum_k X[rows[r], k] * W[n, k] in binary64, k in order.

    X: [M, K] float32, W: [N, K] float32, b: [N] float32.  ``rows`` selects the
    rows of X to compute (default: all).  Returns [len(rows), N] float64.
    """
    X, W, b = _f32(X), _f32(W), _f32(b)
    M, K = X.shape
    N, K2 = W.shape
    if K2 != K or b.shape != (N,):
        raise ValueError("shape mismatch: X %s, W %s, b %s" % (X.shape, W.shape, b.shape))
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row index out of range")
    Y = np.empty((rows.size, N), dtype=np.float64)
    if rows.size and N:
        _load().oracle_linear_rows(M, N, K, _ptr(X), _ptr(W), _ptr(b), _ptr(rows), rows.size, _ptr(Y))
    return Y


def gelu(x) -> np.ndarray:
    """Exact-erf GELU, x * Phi(x), elementwise in binary64."""
    x = _f64(x)
    out = np.empty_like(x)
    _load().oracle_gelu(_ptr(x), x.size, _ptr(out))
    return out


def tail_scale_hardtanh_gelu(y, scale: float, lo: float, hi: float) -> np.ndarray:
    """Tail (a): GELU(hardtanh(y * scale, lo, hi)), elementwise."""
    y = _f64(y)
    out = np.empty_like(y)
    _load().oracle_tail_scale_hardtanh_gelu(_ptr(y), y.size, float(scale), float(lo), float(hi), _ptr(out))
    return out


def avgpool1d(y, kernel: int, stride: int | None = None) -> np.ndarray:
    """AvgPool1d over the last axis of a 2-D array: stride defaults to kernel,
    no padding, floor mode.  Returns [rows, floor((N - kernel) / stride) + 1]."""
    y = _f64(y)
    if y.ndim != 2:
        raise ValueError("avgpool1d expects [rows, N]")
    stride = kernel if stride is None else stride
    rows, N = y.shape
    L = (N - kernel) // stride + 1 if N >= kernel else 0
    out = np.empty((rows, max(L, 0)), dtype=np.float64)
    got = _load().oracle_avgpool1d(_ptr(y), rows, N, int(kernel), int(stride), _ptr(out))
    assert got == L
    return out


def tail_pool_gelu_scale_rowmax(y, kernel: int, scale: float, stride: int | None = None):
    """Tail (b) on [rows, N]: returns (rowmax [rows], g [rows, L], pooled [rows, L]),
    where g = GELU(pooled) * scale is the materialised vector the max runs over."""
    pooled = avgpool1d(y, kernel, stride)
    rows, L = pooled.shape
    g = np.empty_like(pooled)
    out = np.empty(rows, dtype=np.float64)
    _load().oracle_tail_gelu_scale_rowmax(_ptr(pooled), rows, L, float(scale), _ptr(g), _ptr(out))
    return out, g, pooled


def tail_swish_scale(y, scale: float) -> np.ndarray:
    """Tail (c): (y * sigmoid(y)) * scale, elementwise."""
    y = _f64(y)
    out = np.empty_like(y)
    _load().oracle_tail_swish_scale(_ptr(y), y.size, float(scale), _ptr(out))
    return out


# Tail kinds, in the numbering the C interface uses for its epilogue descriptor.
KIND_NONE = 0
KIND_SCALE_HARDTANH_GELU = 1
KIND_POOL_GELU_SCALE_ROWMAX = 2
KIND_SWISH_SCALE = 3
KIND_GELU_SCALE_ROWMAX = 4


def apply_tail(y, kind: int, scale: float = 1.0, lo: float = -1.0, hi: float = 1.0, pool_kernel: int = 16):
    """Apply tail ``kind`` to an already computed linear output y [rows, N]."""
    if kind == KIND_NONE:
        return _f64(y)
    if kind == KIND_SCALE_HARDTANH_GELU:
        return tail_scale_hardtanh_gelu(y, scale, lo, hi)
    if kind == KIND_POOL_GELU_SCALE_ROWMAX:
        return tail_pool_gelu_scale_rowmax(y, pool_kernel, scale)[0]
    if kind == KIND_SWISH_SCALE:
        return tail_swish_scale(y, scale)
    if kind == KIND_GELU_SCALE_ROWMAX:
        # tail (b) with a window of one column: the row max of scale*GELU(y)
        return tail_pool_gelu_scale_rowmax(y, 1, scale)[0]
    raise ValueError("unknown tail kind %r" % kind)


def forward_rows(X, W, b, kind: int, rows=None, **tail):
    """The whole layer for the selected rows: linear, then the tail, unfused."""
    return apply_tail(linear_rows(X, W, b, rows), kind, **tail)
