"""Properties of the planner over random shapes, tails and options.

lin_epi_query_plan with an explicit compute-unit count is a pure host
computation (no GPU), so these run on the CPU.  Every plan must be one the
kernels can run: a tile from the table, a split within the K steps, a grid
that matches its schedule (one tile per workgroup, S segments per tile, or a
stream-K grid within one round of resident workgroups), one kernel per call
except the weight-streaming row-max pass, and a workspace that holds the
intermediates the plan reports."""

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import dense_linear_layer_amd as lib

ROWMAX = (lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX, lib.LIN_EPI_GELU_SCALE_ROWMAX)
# resident workgroups per CU of each LDS tile
PER_CU = {(256, 256): 1, (128, 256): 1, (128, 128): 2, (64, 64): 4, (32, 128): 4, (64, 128): 3, (128, 96): 2}
DECODE = lib.TILE_CONFIGS[lib.TILE_DECODE]
CUS = 256


@pytest.fixture(scope="module")
def handle():
    rc, h = lib.lin_epi_create(None)
    assert rc == lib.LIN_EPI_OK
    yield h
    lib.lin_epi_destroy(h)


def _cdiv(a, b):
    return -(-a // b)


@st.composite
def problems(draw):
    kind = draw(st.sampled_from([lib.LIN_EPI_NONE, lib.LIN_EPI_SCALE_HARDTANH_GELU, lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX,
                                 lib.LIN_EPI_SWISH_SCALE, lib.LIN_EPI_GELU_SCALE_ROWMAX]))
    M = draw(st.one_of(st.integers(1, 40), st.integers(1, 6000)))
    N = draw(st.integers(16 if kind == lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX else 1, 40000))
    K = 4 * draw(st.one_of(st.integers(0, 20), st.integers(0, 9000)))
    return M, N, K, kind


def _check(p, M, N, K, kind):
    tm, tn = p.tile_m, p.tile_n
    assert (tm, tn) in lib.TILE_CONFIGS.values() and p.tile_k == 32
    steps = max(1, _cdiv(K, 32))
    assert 1 <= p.split_k <= steps
    assert p.grid_main >= 1
    rowmax = kind in ROWMAX
    if (tm, tn) == DECODE:
        # the weight-streaming kernel: 16-row X blocks against 64-row W
        # blocks, split_k K segments each, four wavefront units per workgroup
        units = _cdiv(M, 16) * _cdiv(N, 64) * p.split_k
        assert p.grid_main == _cdiv(units, 4)
        assert p.schedule == (1 if p.split_k > 1 else 0)
        assert p.kernels == (2 if rowmax else 1)
    else:
        tiles = _cdiv(M, tm) * _cdiv(N, tn)
        if p.schedule == 0:
            assert p.grid_main == tiles and p.split_k == 1
        elif p.schedule == 1:
            assert p.grid_main == tiles * p.split_k and p.split_k >= 2
        else:
            assert p.schedule == 2
            assert p.grid_main != tiles and p.grid_main % tiles != 0 and p.grid_main < tiles * steps
        assert p.kernels == 1
        if rowmax:
            assert p.workspace_bytes >= M * _cdiv(N, tn) * 4  # per-tile row maxima
    if p.split_k == 1:
        assert p.partial_bytes == 0
    else:
        assert p.partial_bytes > 0
    if p.split_k == 1 and not rowmax:
        assert p.workspace_bytes == 0
    else:
        assert p.workspace_bytes >= p.partial_bytes > -1


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(problems())
def test_automatic_plans_are_runnable(handle, prob):
    M, N, K, kind = prob
    rc, p = lib.lin_epi_query_plan(handle, M, N, K, lib.make_desc(kind, 1.0), CUS)
    assert rc == lib.LIN_EPI_OK
    _check(p, M, N, K, kind)
    if p.schedule == 2:
        # stream-K grids stay within one round of resident workgroups
        assert p.grid_main <= CUS * PER_CU[(p.tile_m, p.tile_n)]
    rc2, p2 = lib.lin_epi_query_plan(handle, M, N, K, lib.make_desc(kind, 1.0), CUS)
    assert rc2 == lib.LIN_EPI_OK
    assert bytes(p2) == bytes(p), "the planner is deterministic"


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(problems(), st.sampled_from(sorted(lib.TILE_CONFIGS)), st.integers(0, 9), st.sampled_from([0, 0, 1, 7, 256, 700]))
def test_forced_plans_honour_the_options(handle, prob, tile, split, grid):
    M, N, K, kind = prob
    opts = ((lib.LIN_EPI_OPT_TILE, tile), (lib.LIN_EPI_OPT_SPLIT_K, split), (lib.LIN_EPI_OPT_GRID, grid))
    for o, v in opts:
        assert lib.lin_epi_set_option(handle, o, v) == 0
    try:
        rc, p = lib.lin_epi_query_plan(handle, M, N, K, lib.make_desc(kind, 1.0), CUS)
    finally:
        for o, _ in opts:
            assert lib.lin_epi_set_option(handle, o, 0) == 0
    assert rc == lib.LIN_EPI_OK
    _check(p, M, N, K, kind)
    assert (p.tile_m, p.tile_n) == lib.TILE_CONFIGS[tile]
    steps = max(1, _cdiv(K, 32))
    if (p.tile_m, p.tile_n) != DECODE:
        tiles = _cdiv(M, p.tile_m) * _cdiv(N, p.tile_n)
        if grid > 0:
            # a forced grid, clamped to the (tile, K step) work
            assert p.grid_main == min(grid, tiles * steps)
        elif split == 1:
            assert p.grid_main == tiles and p.split_k == 1
        elif split >= 2:
            assert p.split_k == min(split, steps)
