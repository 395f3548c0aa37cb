"""GPU parity of the weight-streaming kernel (tile option 6): few rows of X
against a long stream of W rows, operands loaded from HBM straight into a
register ring, K segments added by the last wavefront of each block to
finish.  Integer inputs compare bit for bit with the oracle; random inputs
compare to 1e-3 * (1 + |ref|) and rerun bitwise."""

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


@pytest.mark.parametrize("split", [1, 2, 3, 7])
@pytest.mark.parametrize("M,N,K", [(1, 1, 4), (1, 33, 36), (5, 100, 1028), (16, 4096, 4100), (17, 77, 260),
                                   (33, 530, 1000), (16, 31, 32), (9, 1000, 8)])
def test_decode_integer_exact(M, N, K, split):
    """Ragged in every dimension (M past one 16-row block, N past a 32-row W
    block, K % 32 != 0 so the first K step is partial), segments 1..7."""
    X, W, b = workloads.integer_inputs(M, N, K, seed=M * 7 + N + K + split)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, lib.TILE_DECODE)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
        p = h.plan()
        assert (p.tile_m, p.tile_n) == (16, 64)
        assert p.split_k == min(split, -(-K // 32))
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))


@pytest.mark.parametrize("split", [1, 4])
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_decode_all_tails(tail, split):
    """Every tail through the weight-streaming kernel on a ragged few-row
    layer (N = 6000 gives 375 whole pooling windows and a last W block with a
    partial window), reruns bitwise identical."""
    M, N, K = 7, 6000, 4100
    X, W, b = workloads.make_inputs(M, N, K, seed=split + 3)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, lib.TILE_DECODE)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        assert p.kernels == (2 if tail.kind in ROWMAX else 1)
        compare(got, oracle_rows(X, W, b, tail), what="decode split %d %s" % (split, tail.name))
        for _ in range(2):
            assert np.array_equal(run_gpu(h, Xd, Wd, bd, tail), got), "decode rerun not bitwise identical"


@pytest.mark.parametrize("M", [1, 2, 8, 16])
def test_planner_picks_decode_for_few_rows(M):
    """For a handful of rows against a large weight the planner streams W
    with the weight-streaming kernel; checked against the oracle."""
    N, K = 8192, 8192
    X, W, b = workloads.make_inputs(M, N, K, seed=M)
    with lib.LinEpi() as h:
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_C)
        p = h.plan()
        log("plan: tile %dx%d split %d grid %d" % (p.tile_m, p.tile_n, p.split_k, p.grid_main))
        assert (p.tile_m, p.tile_n) == (16, 64)
    compare(got, oracle_rows(X, W, b, workloads.TAIL_C), what="M=%d planner" % M)


def test_decode_counters_clean_after_mixed_runs():
    """Split runs of the weight-streaming kernel and of an MFMA tile kernel
    on one handle share the workspace's arrival counters; every run must
    leave them at zero (else the next run finishes blocks early)."""
    cases = [((5, 700, 1028), dict(tile=6, split=5)), ((300, 530, 1028), dict(tile=4, grid=301)),
             ((5, 700, 1028), dict(tile=6, split=3)), ((16, 2000, 4100), dict(tile=6, split=16)),
             ((5, 700, 1028), dict(tile=6, split=5))]
    with lib.LinEpi() as h:
        for (M, N, K), opt in cases:
            X, W, b = workloads.integer_inputs(M, N, K, seed=M + N + K)
            h.set_option(lib.LIN_EPI_OPT_TILE, opt.get("tile", 0))
            h.set_option(lib.LIN_EPI_OPT_GRID, opt.get("grid", 0))
            h.set_option(lib.LIN_EPI_OPT_SPLIT_K, opt.get("split", 0))
            got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
            assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b)), "%s %s" % ((M, N, K), opt)
