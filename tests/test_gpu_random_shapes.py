"""Seeded random problems against the CPU oracle: shapes ragged in every
dimension (K a multiple of 4, as the C ABI requires), every tail, and the
tile configuration and K split either left to the planner or forced, so the
direct-to-LDS and register-staged paths, the swizzled layouts of every tile
and the split-K passes meet many edge combinations.  The cases are drawn once
from a fixed seed, so each one is reproducible by its id."""

import numpy as np
import pytest

import dense_linear_layer_amd as lib
import workloads
from parity_util import compare, log, oracle_rows, run_gpu, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALL_TAILS = (workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C, workloads.TAIL_NONE, workloads.TAIL_B_FOLDED)


def _cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        tail = ALL_TAILS[i % len(ALL_TAILS)]
        M = int(rng.integers(1, 300))
        N = int(rng.integers(16 if tail.kind == workloads.POOL_GELU_SCALE_ROWMAX else 1, 700))
        K = 4 * int(rng.integers(0, 300))
        tile = int(rng.integers(0, 6))            # 0 = planner's choice
        split = int(rng.choice([0, 1, 2, 3, 5]))  # 0 = planner's choice
        reg = bool(rng.integers(0, 4) == 0)       # register staging on a quarter of the cases
        out.append(pytest.param(M, N, K, tail, tile, split, reg,
                                id="%d-%dx%dx%d-%s-t%d-s%d%s" % (i, M, N, K, tail.name, tile, split, "-reg" if reg else "")))
    return out


@pytest.fixture(autouse=True)
def _name(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log("== %s" % request.node.nodeid)


@pytest.mark.parametrize("M,N,K,tail,tile,split,reg", _cases())
def test_random_problem_matches_oracle(M, N, K, tail, tile, split, reg):
    X, W, b = workloads.make_inputs(M, N, K, seed=M * 7919 + N * 31 + K)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        h.set_option(lib.LIN_EPI_OPT_REG_STAGING, int(reg))
        got = run_gpu(h, *to_dev(X, W, b), tail)
        p = h.plan()
        if tile:
            assert (p.tile_m, p.tile_n) == lib.TILE_CONFIGS[tile]
    compare(got, oracle_rows(X, W, b, tail),
            what="%dx%dx%d %s tile %dx%d split %d%s" % (M, N, K, tail.name, p.tile_m, p.tile_n, p.split_k,
                                                       " reg" if reg else ""))
