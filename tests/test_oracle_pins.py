"""Pins for the CPU oracle: things the pages and the mathematics fix, checked
without reference to the oracle's own formulas.

Each group targets a plausible mistake: a transposed operand or wrong index
in the linear layer (brute force on non-square shapes, identity inputs,
row selection), a dropped bias (zero input), the wrong GELU (closed forms
that separate exact-erf from the tanh approximation), a wrong op order or
sign in a tail (hand-picked points where the orders differ, odd-part
identities), wrong pooling (the page's worked example, constant windows,
window-count formula), and GELU hoisted past the max (a case where GELU's
non-monotonicity changes the answer).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import optimize, special, stats

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# GELU's global minimum, from the closed form GELU'(x) = Phi(x) + x*phi(x) = 0
# solved to 1e-12 with a bracketing root finder on the library CDF/PDF.
_XMIN = optimize.brentq(lambda x: stats.norm.cdf(x) + x * stats.norm.pdf(x), -1.0, -0.5, xtol=1e-14)
GELU_MIN = _XMIN * stats.norm.cdf(_XMIN)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Linear layer y = x W^T + b
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 4, 5), (7, 33, 5), (2, 3, 17), (5, 2, 1)])
def test_linear_brute_force_exact(M, N, K):
    """Exact rational arithmetic on tiny non-square shapes: any transposed
    operand, wrong stride or dropped bias changes the result."""
    X, W, b = workloads.make_inputs(M, N, K, seed=M * 100 + N * 10 + K)
    y = oracle.linear_rows(X, W, b)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(X[m, k])) * Fraction(float(W[n, k])) for k in range(K)), Fraction(0))
            exact += Fraction(float(b[n]))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10**12) * (1 + abs(exact))


@pytest.mark.parametrize("M,N,K,seed", [(64, 48, 40, 1), (13, 64, 29, 2), (1, 17, 64, 3), (33, 1, 7, 4)])
def test_linear_matches_library_matmul(M, N, K, seed):
    X, W, b = workloads.make_inputs(M, N, K, seed=seed)
    ref = X.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(oracle.linear_rows(X, W, b), ref, rtol=1e-13, atol=1e-13)


def test_linear_identity_input_gives_weight_transpose():
    K, N = 24, 37
    _, W, b = workloads.make_inputs(1, N, K, seed=5)
    X = np.eye(K, dtype=np.float32)
    y = oracle.linear_rows(X, W, b)
    assert np.array_equal(y, W.T.astype(np.float64) + b.astype(np.float64))


def test_linear_zero_input_gives_bias():
    _, W, b = workloads.make_inputs(1, 19, 11, seed=6)
    X = np.zeros((5, 11), dtype=np.float32)
    y = oracle.linear_rows(X, W, b)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), (5, 19)))


def test_linear_zero_k_gives_bias():
    W = np.zeros((4, 0), dtype=np.float32)
    b = np.arange(4, dtype=np.float32)
    y = oracle.linear_rows(np.zeros((3, 0), dtype=np.float32), W, b)
    assert np.array_equal(y, np.tile(b.astype(np.float64), (3, 1)))


def test_linear_integer_inputs_exact():
    X, W, b = workloads.integer_inputs(9, 21, 4100, seed=7)
    y = oracle.linear_rows(X, W, b)
    ref = X.astype(np.int64) @ W.astype(np.int64).T + b.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64))


def test_linear_row_subset_selects_rows():
    X, W, b = workloads.make_inputs(20, 6, 9, seed=8)
    rows = np.array([19, 0, 7], dtype=np.int64)
    full = oracle.linear_rows(X, W, b)
    assert np.array_equal(oracle.linear_rows(X, W, b, rows), full[rows])


# --------------------------------------------------------------------------
# GELU (exact erf)
# --------------------------------------------------------------------------

def test_gelu_table_values():
    """GELU(x) = x * Phi(x) at textbook table points; the tanh approximation
    misses GELU(2) by ~1e-4, far above this tolerance."""
    g = _golden("gelu_points.json")["phi_cdf_table"]
    x = np.array(g["x"])
    np.testing.assert_allclose(oracle.gelu(x), x * np.array(g["Phi"]), rtol=0, atol=1e-14)
    tanh_form = 0.5 * 2.0 * (1 + math.tanh(math.sqrt(2 / math.pi) * (2.0 + 0.044715 * 8.0)))
    assert abs(oracle.gelu([2.0])[0] - tanh_form) > 5e-5


def test_gelu_matches_normal_cdf_library():
    x = np.linspace(-12, 12, 2001)
    np.testing.assert_allclose(oracle.gelu(x), x * stats.norm.cdf(x), rtol=1e-13, atol=1e-15)


def test_gelu_closed_forms():
    assert oracle.gelu([0.0])[0] == 0.0
    x = np.linspace(-6, 6, 241)
    # odd-part identity: GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1)
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, atol=1e-14)
    # GELU(x) -> x for large positive x, -> 0 for large negative x
    assert abs(oracle.gelu([10.0])[0] - 10.0) < 1e-15 * 10
    assert abs(oracle.gelu([-10.0])[0]) < 1e-20


def test_gelu_derivative_at_minus_one_matches_page():
    g = _golden("gelu_points.json")
    h = 1e-6
    d = (oracle.gelu([-1 + h])[0] - oracle.gelu([-1 - h])[0]) / (2 * h)
    assert abs(d - g["derivative_at_minus_one"]) < g["derivative_tolerance"]
    # closed form Phi(-1) - phi(-1)
    assert abs(d - (stats.norm.cdf(-1) - stats.norm.pdf(-1))) < 1e-8


def test_gelu_global_minimum():
    res = optimize.minimize_scalar(lambda t: oracle.gelu([t])[0], bounds=(-3, 0), method="bounded",
                                   options={"xatol": 1e-10})
    assert abs(res.x - _XMIN) < 1e-6
    assert abs(res.fun - GELU_MIN) < 1e-12
    assert abs(GELU_MIN - (-0.16997120)) < 1e-7


# --------------------------------------------------------------------------
# Tail (a): scale -> hardtanh -> GELU
# --------------------------------------------------------------------------

def test_tail_a_op_order_and_saturation():
    s, lo, hi = 0.5, -2.0, 2.0
    y = np.array([0.0, 3.0, -3.0, 4.0, 5.0, -4.0, -100.0, 100.0, 1.0])
    out = oracle.tail_scale_hardtanh_gelu(y, s, lo, hi)
    phi2 = 0.9772498680518208
    gelu2, gelum2 = 2.0 * phi2, -2.0 * (1 - phi2)
    # y=3: scale first gives t=1.5 (inside); clamping first would give GELU(1).
    assert abs(out[1] - 1.5 * stats.norm.cdf(1.5)) < 1e-14
    assert abs(out[2] - (-1.5) * stats.norm.cdf(-1.5)) < 1e-14
    # y*s == +-2 exactly sits on the clamp; beyond it saturates at GELU(+-2)
    for i in (3, 4, 7):
        assert abs(out[i] - gelu2) < 1e-14
    for i in (5, 6):
        assert abs(out[i] - gelum2) < 1e-14
    assert out[0] == 0.0
    assert abs(out[8] - 0.5 * stats.norm.cdf(0.5)) < 1e-14


def test_tail_a_range_bounds():
    y = np.random.default_rng(9).normal(0, 8, 100000)
    out = oracle.tail_scale_hardtanh_gelu(y, 0.5, -2.0, 2.0)
    assert out.max() <= 2 * 0.9772498680518208 + 1e-15
    assert out.min() >= GELU_MIN - 1e-15


def test_tail_a_asymmetric_clamp():
    # a clamp [-1, 3] with scale 2: y=1 -> t=2 inside; y=-1 -> t=-2 clamps to -1
    out = oracle.tail_scale_hardtanh_gelu(np.array([1.0, -1.0, 2.0]), 2.0, -1.0, 3.0)
    np.testing.assert_allclose(out, [2 * stats.norm.cdf(2), -stats.norm.cdf(-1), 3 * stats.norm.cdf(3)], atol=1e-14)


# --------------------------------------------------------------------------
# Tail (b): AvgPool1d(k) -> GELU -> scale -> row max
# --------------------------------------------------------------------------

def test_pool_worked_example_from_page():
    g = _golden("pool_fold_worked_example.json")
    X = np.array(g["x"], dtype=np.float32)
    W = np.array(g["W"], dtype=np.float32)
    b = np.array(g["b"], dtype=np.float32)
    y = oracle.linear_rows(X, W, b)
    assert np.array_equal(y, np.array(g["linear"]))
    pooled = oracle.avgpool1d(y, g["pool_kernel"])
    assert np.array_equal(pooled, np.array(g["pooled"]))
    # fold identity of the same passage: pool the weights, then the linear layer
    Wp = oracle.avgpool1d(W.T.astype(np.float64), g["pool_kernel"]).T
    assert np.array_equal(Wp, np.array(g["pooled_weight"]))
    bp = oracle.avgpool1d(b[None, :].astype(np.float64), g["pool_kernel"])[0]
    folded = oracle.linear_rows(X, Wp.astype(np.float32), bp.astype(np.float32))
    assert np.array_equal(folded, pooled)


@pytest.mark.parametrize("N,k,L", [(8192, 16, 512), (6000, 16, 375), (15, 16, 0), (16, 16, 1), (35, 16, 2), (4, 2, 2)])
def test_pool_output_width(N, k, L):
    assert oracle.avgpool1d(np.zeros((2, N)), k).shape == (2, L)


def test_pool_matches_reshape_mean_and_ignores_tail_columns():
    y = np.random.default_rng(10).normal(size=(3, 16 * 7 + 5))
    ref = y[:, : 16 * 7].reshape(3, 7, 16).mean(axis=2)
    np.testing.assert_allclose(oracle.avgpool1d(y, 16), ref, rtol=1e-14, atol=1e-15)
    y2 = y.copy()
    y2[:, 16 * 7:] = 1e9  # trailing N % 16 columns never reach a window
    assert np.array_equal(oracle.avgpool1d(y2, 16), oracle.avgpool1d(y, 16))


def test_pool_constant_window_is_the_constant():
    vals = np.array([0.375, -1.25, 7.0, 0.0])  # dyadic: the window sums are exact
    y = np.repeat(vals, 16)[None, :]
    assert np.array_equal(oracle.avgpool1d(y, 16)[0], vals)
    y = np.full((1, 32), 0.3)
    np.testing.assert_allclose(oracle.avgpool1d(y, 16)[0], [0.3, 0.3], rtol=1e-15)


def test_tail_b_gelu_before_max():
    """GELU is not monotonic (page l2_p98), so max of GELU differs from GELU of max."""
    y = np.concatenate([np.full(16, _XMIN), np.full(16, -3.0)])[None, :]
    out, g, pooled = oracle.tail_pool_gelu_scale_rowmax(y, 16, 2.0)
    np.testing.assert_allclose(pooled[0], [_XMIN, -3.0], atol=1e-15)
    expect = 2.0 * (-3.0) * stats.norm.cdf(-3.0)
    assert abs(out[0] - expect) < 1e-14
    assert abs(out[0] - 2.0 * GELU_MIN) > 0.3  # the hoisted order would give this


def test_tail_b_scale_after_gelu_and_invariants():
    y = np.random.default_rng(11).normal(0, 0.6, size=(40, 16 * 33))
    out, g, pooled = oracle.tail_pool_gelu_scale_rowmax(y, 16, 2.0)
    np.testing.assert_allclose(g, 2.0 * pooled * stats.norm.cdf(pooled), rtol=1e-13, atol=1e-15)
    assert np.array_equal(out, g.max(axis=1))
    assert (out >= 2.0 * GELU_MIN - 1e-15).all()


def test_fold_identity_on_random_layer():
    X, W, b = workloads.make_inputs(6, 64, 20, seed=12)
    pooled = oracle.avgpool1d(oracle.linear_rows(X, W, b), 16)
    Wp = W.astype(np.float64).reshape(4, 16, 20).mean(axis=1)
    bp = b.astype(np.float64).reshape(4, 16).mean(axis=1)
    folded = X.astype(np.float64) @ Wp.T + bp
    np.testing.assert_allclose(pooled, folded, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Tail (c): swish -> scale
# --------------------------------------------------------------------------

def test_swish_closed_forms():
    y = np.linspace(-30, 30, 1201)
    out = oracle.tail_swish_scale(y, 2.0)
    np.testing.assert_allclose(out, 2.0 * y * special.expit(y), rtol=1e-13, atol=1e-300)
    assert oracle.tail_swish_scale(np.array([0.0]), 2.0)[0] == 0.0
    one = oracle.tail_swish_scale(y, 1.0)
    np.testing.assert_allclose(one - oracle.tail_swish_scale(-y, 1.0), y, atol=1e-13)
    assert abs(oracle.tail_swish_scale(np.array([40.0]), 2.0)[0] - 80.0) < 1e-12
    assert abs(oracle.tail_swish_scale(np.array([-40.0]), 2.0)[0]) < 1e-14


def test_swish_minimum_lambert_w():
    w = special.lambertw(math.exp(-1)).real
    xstar = -1.0 - w
    res = optimize.minimize_scalar(lambda t: oracle.tail_swish_scale(np.array([t]), 2.0)[0], bounds=(-4, 0),
                                   method="bounded", options={"xatol": 1e-10})
    assert abs(res.x - xstar) < 1e-6
    assert abs(res.fun - 2.0 * (xstar + 1.0)) < 1e-12
    assert abs(2.0 * (xstar + 1.0) - (-0.55692909)) < 1e-8


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def test_forward_rows_composes_linear_and_tail():
    X, W, b = workloads.make_inputs(10, 48, 12, seed=13)
    rows = np.array([2, 9])
    y = X.astype(np.float64)[rows] @ W.astype(np.float64).T + b
    np.testing.assert_allclose(oracle.forward_rows(X, W, b, oracle.KIND_SWISH_SCALE, rows, scale=2.0),
                               2.0 * y * special.expit(y), rtol=1e-12)
    rm = oracle.forward_rows(X, W, b, oracle.KIND_POOL_GELU_SCALE_ROWMAX, rows, scale=2.0, pool_kernel=16)
    p = y.reshape(2, 3, 16).mean(axis=2)
    np.testing.assert_allclose(rm, (2.0 * p * stats.norm.cdf(p)).max(axis=1), rtol=1e-12)


def test_workload_value_structure():
    """The recipe gives y ~ N(0, 1/3) whatever K (Var = K * TK^2 / 3)."""
    X, W, b = workloads.make_inputs(64, 512, 2048, seed=0)
    y = oracle.linear_rows(X, W, b)
    assert abs(y.std() - math.sqrt(1 / 3)) < 0.02
    assert np.abs(W).max() <= workloads.bound(2048)


def test_checked_rows():
    r = workloads.checked_rows(2048)
    assert r.size == 64 and r[0] == 0 and r[-1] == 2047 and np.unique(r).size == 64
    assert np.array_equal(r, workloads.checked_rows(2048))
    assert np.array_equal(workloads.checked_rows(40), np.arange(40))


# --------------------------------------------------------------------------
# Dispatch: forward_rows / apply_tail, the route every GPU parity test takes.
# Each kind is pinned through that route, so a mistake in the dispatch itself
# (arguments swapped or dropped, the wrong window) fails here too.
# --------------------------------------------------------------------------

def _column_layer(values):
    """X = I_K, W = values as one output feature, b = 0: the linear output of
    row m is values[m] exactly, so forward_rows exposes the tail alone."""
    v = np.asarray(values, dtype=np.float32)
    X = np.eye(v.size, dtype=np.float32)
    return X, v[None, :].copy(), np.zeros(1, dtype=np.float32)


def test_dispatch_kind0_is_the_linear_layer():
    K, N = 24, 37
    _, W, b = workloads.make_inputs(1, N, K, seed=14)
    X = np.eye(K, dtype=np.float32)
    y = oracle.forward_rows(X, W, b, oracle.KIND_NONE, scale=3.0, lo=-0.5, hi=0.5)
    assert np.array_equal(y, W.T.astype(np.float64) + b.astype(np.float64))
    rows = np.array([5, 0, 23])
    assert np.array_equal(oracle.forward_rows(X, W, b, oracle.KIND_NONE, rows), y[rows])


def test_dispatch_kind1_op_order_and_saturation():
    """The points of the tail (a) closed-form pin, run through forward_rows."""
    X, W, b = _column_layer([0.0, 3.0, -3.0, 4.0, 5.0, -4.0, -100.0, 100.0, 1.0])
    out = oracle.forward_rows(X, W, b, oracle.KIND_SCALE_HARDTANH_GELU, scale=0.5, lo=-2.0, hi=2.0)[:, 0]
    phi2 = 0.9772498680518208
    assert out[0] == 0.0
    assert abs(out[1] - 1.5 * stats.norm.cdf(1.5)) < 1e-14     # scale before the clamp
    assert abs(out[2] - (-1.5) * stats.norm.cdf(-1.5)) < 1e-14
    for i in (3, 4, 7):
        assert abs(out[i] - 2.0 * phi2) < 1e-14                # saturates at GELU(2)
    for i in (5, 6):
        assert abs(out[i] - (-2.0) * (1 - phi2)) < 1e-14       # and at GELU(-2)
    assert abs(out[8] - 0.5 * stats.norm.cdf(0.5)) < 1e-14


def test_dispatch_kind1_asymmetric_clamp():
    """lo and hi reach the clamp in that order: [-1, 3] with scale 2."""
    X, W, b = _column_layer([1.0, -1.0, 2.0])
    out = oracle.forward_rows(X, W, b, oracle.KIND_SCALE_HARDTANH_GELU, scale=2.0, lo=-1.0, hi=3.0)[:, 0]
    np.testing.assert_allclose(out, [2 * stats.norm.cdf(2), -stats.norm.cdf(-1), 3 * stats.norm.cdf(3)], atol=1e-14)


def test_dispatch_kind2_worked_example_window():
    """The page's worked example (window 2) through forward_rows: the row max
    of 2*GELU over the pooled values [1.5, 4.5]."""
    g = _golden("pool_fold_worked_example.json")
    X = np.array(g["x"], dtype=np.float32)
    W = np.array(g["W"], dtype=np.float32)
    b = np.array(g["b"], dtype=np.float32)
    out = oracle.forward_rows(X, W, b, oracle.KIND_POOL_GELU_SCALE_ROWMAX, scale=2.0, pool_kernel=g["pool_kernel"])
    p = np.array(g["pooled"][0])
    assert abs(out[0] - (2.0 * p * stats.norm.cdf(p)).max()) < 1e-14


def _window_mean_rows(a, k):
    """Mean of each run of k consecutive rows (exact here: dyadic data)."""
    a = np.asarray(a, dtype=np.float64)
    L = a.shape[0] // k
    return a[: L * k].reshape((L, k) + a.shape[1:]).mean(axis=1)


@pytest.mark.parametrize("M,N,K,seed", [(6, 64, 20, 15), (9, 16 * 7 + 5, 12, 16)])
def test_dispatch_kind4_fold_identity(M, N, K, seed):
    """Page l2_p98's fold identity: tail (b) of the layer equals kind 4 (no
    pooling) on the layer with window-averaged weights and bias.  Integer
    inputs make both linear outputs exact, so the two sides agree to 1e-12."""
    X, W, b = workloads.integer_inputs(M, N, K, seed=seed)
    Wp = _window_mean_rows(W, 16).astype(np.float32)
    bp = _window_mean_rows(b, 16).astype(np.float32)
    assert np.array_equal(Wp.astype(np.float64), _window_mean_rows(W, 16))  # exact in fp32
    direct = oracle.apply_tail(oracle.linear_rows(X, W, b), oracle.KIND_POOL_GELU_SCALE_ROWMAX, 2.0)
    folded = oracle.apply_tail(oracle.linear_rows(X, Wp, bp), oracle.KIND_GELU_SCALE_ROWMAX, 2.0)
    assert folded.shape == (M,)
    np.testing.assert_allclose(folded, direct, rtol=0, atol=1e-12)
    via_rows = oracle.forward_rows(X, Wp, bp, oracle.KIND_GELU_SCALE_ROWMAX, scale=2.0)
    assert np.array_equal(via_rows, folded)


def test_dispatch_kind4_is_rowmax_of_scaled_gelu():
    # one row, three output features with linear outputs -0.75, 0.25, -3
    Xr = np.ones((1, 1), dtype=np.float32)
    Wr = np.array([[-0.75], [0.25], [-3.0]], dtype=np.float32)
    br = np.zeros(3, dtype=np.float32)
    out = oracle.forward_rows(Xr, Wr, br, oracle.KIND_GELU_SCALE_ROWMAX, scale=2.0)
    v = np.array([-0.75, 0.25, -3.0])
    assert out.shape == (1,)
    assert abs(out[0] - (2.0 * v * stats.norm.cdf(v)).max()) < 1e-14
