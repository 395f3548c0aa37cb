"""GPU parity of the work partition: split-K and stream-K grids (tiles cut
into K segments that the last-arriving workgroup adds in K order), the K
step grid whose only partial step is the first, and the arrival counters
that every run must leave at zero.  Integer inputs make every partial sum
exact, so those cases compare bit for bit; the others compare with the
oracle to 1e-3 * (1 + |ref|) and rerun bitwise."""

import numpy as np
import pytest

import dense_linear_layer_amd as lib
import oracle
import workloads
from parity_util import compare, log, oracle_rows, run_gpu, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALL_TAILS = (workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C, workloads.TAIL_NONE, workloads.TAIL_B_FOLDED)
ROWMAX = (workloads.POOL_GELU_SCALE_ROWMAX, workloads.GELU_SCALE_ROWMAX)


@pytest.fixture(autouse=True)
def _name(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log("== %s" % request.node.nodeid)


@pytest.mark.parametrize("grid", [1, 5, 37, 256, 301, 512])
@pytest.mark.parametrize("tile", sorted(t for t in lib.TILE_CONFIGS if t != lib.TILE_DECODE))
def test_stream_k_integer_exact(tile, grid):
    """Forced stream-K grids on a shape ragged in M, N and K (K % 32 != 0,
    so the first K step of every tile is the partial one): bit-exact."""
    M, N, K = 300, 530, 1028
    X, W, b = workloads.integer_inputs(M, N, K, seed=tile * 1000 + grid)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_GRID, grid)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
        p = h.plan()
        log("plan: tile %dx%d grid %d schedule %d max segments %d" % (p.tile_m, p.tile_n, p.grid_main, p.schedule,
                                                                     p.split_k))
        tm, tn = lib.TILE_CONFIGS[tile]
        work = -(-M // tm) * -(-N // tn) * -(-K // 32)  # (tile, K step) iterations
        assert p.grid_main == min(grid, work) and (p.tile_m, p.tile_n) == (tm, tn)
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))


@pytest.mark.parametrize("grid", [7, 300])
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_stream_k_all_tails_deterministic(tail, tile, grid):
    M, N, K = 261, 1040, 2084
    X, W, b = workloads.make_inputs(M, N, K, seed=grid + 10 * tile)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_GRID, grid)
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        assert p.kernels == 1  # row maxima too are finished in the tile kernel
        compare(got, oracle_rows(X, W, b, tail), what="stream-K tile %d grid %d %s" % (tile, grid, tail.name))
        for _ in range(2):
            assert np.array_equal(run_gpu(h, Xd, Wd, bd, tail), got), "stream-K rerun not bitwise identical"


@pytest.mark.parametrize("K", [4, 12, 28, 32, 36, 100, 1028, 4100])
@pytest.mark.parametrize("split", [1, 2, 3])
@pytest.mark.parametrize("tile", sorted(lib.TILE_CONFIGS))
def test_first_step_partial_k_integer_exact(tile, split, K):
    """K not a multiple of 32 shifts the K grid so that only step 0 is
    partial (its first 32 - K % 32 positions are zero-filled); with split-K
    only the first segment of a tile holds it."""
    M, N = 70, 150
    X, W, b = workloads.integer_inputs(M, N, K, seed=K + 7 * split + 100 * tile)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))


def test_counters_stay_clean_across_plans():
    """One handle, alternating plans whose workspaces overlap differently: a
    split plan with many tiles (its counters cover a long prefix), a
    row-max plan without split (its per-tile maxima start right after a short
    counter prefix, over the earlier counters), then the first plan again,
    and a split plan with few tiles.  Every run must match the oracle."""
    cases = [
        ((300, 530, 1028), workloads.TAIL_NONE, dict(tile=4, grid=301)),
        ((500, 3000, 100), workloads.TAIL_B, dict(tile=4, split=1)),
        ((300, 530, 1028), workloads.TAIL_NONE, dict(tile=4, grid=301)),
        ((64, 64, 4100), workloads.TAIL_A, dict(tile=3, split=5)),
        ((300, 530, 1028), workloads.TAIL_NONE, dict(tile=4, grid=301)),
    ]
    inputs = {}
    with lib.LinEpi() as h:
        for (M, N, K), tail, opt in cases:
            if (M, N, K) not in inputs:
                X, W, b = workloads.integer_inputs(M, N, K, seed=M + N + K)
                inputs[(M, N, K)] = (X, W, b, to_dev(X, W, b))
            X, W, b, dev = inputs[(M, N, K)]
            h.set_option(lib.LIN_EPI_OPT_TILE, opt.get("tile", 0))
            h.set_option(lib.LIN_EPI_OPT_GRID, opt.get("grid", 0))
            h.set_option(lib.LIN_EPI_OPT_SPLIT_K, opt.get("split", 0))
            got = run_gpu(h, *dev, tail)
            ref = oracle_rows(X, W, b, tail)
            if tail.kind == workloads.NONE:
                assert np.array_equal(got.astype(np.float64), ref), "%s %s" % ((M, N, K), opt)
            else:
                compare(got, ref, what="%s %s %s" % ((M, N, K), tail.name, opt))


@pytest.mark.parametrize("tail", [workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C], ids=lambda t: t.name)
def test_planner_choice_ragged_full_size(tail):
    """The ragged 1000x6000x4100 layer in the plan the benchmark times, all
    rows checked (the oracle runs all 1000 rows in a few seconds)."""
    w = workloads.WORKLOADS["ragged_1000x6000x4100"]
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        log("plan: tile %dx%d grid %d schedule %d segments %d" % (p.tile_m, p.tile_n, p.grid_main, p.schedule,
                                                                 p.split_k))
        assert np.array_equal(run_gpu(h, Xd, Wd, bd, tail), got)
    compare(got, oracle_rows(X, W, b, tail), what="ragged %s" % tail.name)


def _random_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        tail = ALL_TAILS[i % len(ALL_TAILS)]
        M = int(rng.integers(1, 400))
        N = int(rng.integers(16 if tail.kind == workloads.POOL_GELU_SCALE_ROWMAX else 1, 900))
        K = 4 * int(rng.integers(1, 400))
        tile = int(rng.integers(1, 6))
        grid = int(rng.integers(1, 700))
        out.append(pytest.param(M, N, K, tail, tile, grid, id="%d-%dx%dx%d-%s-t%d-g%d" % (i, M, N, K, tail.name, tile,
                                                                                          grid)))
    return out


@pytest.mark.parametrize("M,N,K,tail,tile,grid", _random_cases())
def test_random_stream_k_matches_oracle(M, N, K, tail, tile, grid):
    X, W, b = workloads.make_inputs(M, N, K, seed=M * 131 + N * 7 + K)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_GRID, grid)
        got = run_gpu(h, *to_dev(X, W, b), tail)
        p = h.plan()
    compare(got, oracle_rows(X, W, b, tail), what="%dx%dx%d %s tile %dx%d grid %d" % (M, N, K, tail.name, p.tile_m,
                                                                                      p.tile_n, p.grid_main))


def test_row_max_finish_across_shapes_one_handle():
    """The row-max tails finish in the tile kernel: the last workgroup of
    each tile row to arrive (one device-scope counter per tile row, after the
    per-tile counters in the workspace) takes the max over the row's per-tile
    partials.  One handle, so one workspace, runs shapes whose tile-row and
    column-tile counts grow and shrink (more than 64 column tiles, where a
    lane takes several; a single one), whole-tile and stream-K; each result
    matches the oracle and reruns bitwise, so every run left its counters
    at zero."""
    cases = [
        (300, 5000, 260, workloads.TAIL_B, 4, 0),        # 5 x 79 tiles of 64x64
        (1000, 300, 516, workloads.TAIL_B_FOLDED, 5, 0),  # 32 x 3 tiles of 32x128
        (70, 16, 36, workloads.TAIL_B, 3, 0),             # one column tile
        (300, 5000, 260, workloads.TAIL_B, 4, 301),      # stream-K, 79 column tiles
        (513, 2100, 1028, workloads.TAIL_B_FOLDED, 7, 0),
        (129, 4100, 300, workloads.TAIL_B, 0, 0),         # the planner's choice
        (300, 5000, 260, workloads.TAIL_B, 4, 0),
    ]
    with lib.LinEpi() as h:
        for M, N, K, tail, tile, grid in cases:
            log("case %dx%dx%d %s tile %d grid %d" % (M, N, K, tail.name, tile, grid))
            X, W, b = workloads.make_inputs(M, N, K, seed=M + N + K + grid)
            Xd, Wd, bd = to_dev(X, W, b)
            h.set_option(lib.LIN_EPI_OPT_TILE, tile)
            h.set_option(lib.LIN_EPI_OPT_GRID, grid)
            got = run_gpu(h, Xd, Wd, bd, tail)
            p = h.plan()
            assert p.kernels == 1 and (p.tile_m, p.tile_n) != lib.TILE_CONFIGS[lib.TILE_DECODE]
            compare(got, oracle_rows(X, W, b, tail), what="%dx%dx%d %s tile %dx%d grid %d" % (
                M, N, K, tail.name, p.tile_m, p.tile_n, p.grid_main))
            assert np.array_equal(run_gpu(h, Xd, Wd, bd, tail), got), "rerun not bitwise identical"


@pytest.mark.parametrize("M,N,K,tail", [(3000, 3000, 3000, workloads.TAIL_A), (768, 3072, 3072, workloads.TAIL_C),
                                        (1536, 1536, 6144, workloads.TAIL_A), (640, 5000, 5000, workloads.TAIL_C)],
                         ids=["3000^3-a", "768x3072x3072-c", "1536x1536x6144-a", "640x5000x5000-c"])
def test_planner_choice_on_128x96_shapes(M, N, K, tail):
    """Shapes where the planner picks the 128x96 tile (a round and a half of
    whole tiles at 3000^3; stream-K over one workgroup per CU for the others):
    64 sampled rows against the oracle, and a bitwise rerun."""
    X, W, b = workloads.make_inputs(M, N, K, seed=M + K)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        log("plan: tile %dx%d grid %d schedule %d segments %d" % (p.tile_m, p.tile_n, p.grid_main, p.schedule,
                                                                 p.split_k))
        assert (p.tile_m, p.tile_n) == (128, 96)
        assert np.array_equal(run_gpu(h, Xd, Wd, bd, tail), got), "rerun not bitwise identical"
    rows = workloads.checked_rows(M, seed=M)
    compare(got[rows], oracle_rows(X, W, b, tail, rows), what="%dx%dx%d %s" % (M, N, K, tail.name))
