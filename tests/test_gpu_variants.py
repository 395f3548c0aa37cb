"""GPU parity of the follow-up variants against the CPU oracle:

* the unfused ablation (LIN_EPI_OPT_UNFUSED): GEMM to memory, then a separate
  tail kernel — must give the same results as the definition;
* the pooled-weight form of tail (b) (lin_epi_pool_weights + kind 4), the
  identity page "Kimi-K2.6 l2_p98" derives and checks on a small example.
"""

import json
import os

import numpy as np
import pytest

import dense_linear_layer_amd as lib
import oracle
import workloads
from parity_util import compare, log, oracle_rows, run_gpu, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL_TAILS = (workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C, workloads.TAIL_NONE, workloads.TAIL_B_FOLDED)


@pytest.fixture(autouse=True)
def _name(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log("== %s" % request.node.nodeid)


# ---------------------------------------------------------------- unfused

@pytest.mark.parametrize("M,N,K", [(5, 48, 12), (130, 290, 100), (257, 1040, 520), (64, 16, 8)])
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_unfused_matches_oracle(M, N, K, tail):
    X, W, b = workloads.make_inputs(M, N, K, seed=7 * M + N)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_UNFUSED, 1)
        got = run_gpu(h, *to_dev(X, W, b), tail)
        p = h.plan()
        assert p.kernels == 1 + (0 if tail.kind == workloads.NONE else 1)
    compare(got, oracle_rows(X, W, b, tail), what="unfused %dx%dx%d %s" % (M, N, K, tail.name))


@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_unfused_with_split_k(tail):
    X, W, b = workloads.make_inputs(200, 390, 1000, seed=71)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_UNFUSED, 1)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 3)
        got = run_gpu(h, *to_dev(X, W, b), tail)
        assert h.plan().split_k == 3
    compare(got, oracle_rows(X, W, b, tail), what="unfused split-3 %s" % tail.name)


def test_unfused_equals_fused_on_integer_inputs():
    """Integer inputs make the GEMM exact, so the raw outputs of both paths are
    identical and the tails see the same arguments."""
    X, W, b = workloads.integer_inputs(300, 520, 260, seed=72)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        fused = run_gpu(h, Xd, Wd, bd, workloads.TAIL_NONE)
        h.set_option(lib.LIN_EPI_OPT_UNFUSED, 1)
        unfused = run_gpu(h, Xd, Wd, bd, workloads.TAIL_NONE)
    assert np.array_equal(fused, unfused)


# ------------------------------------------------------ pooled weights (f1)

def test_pool_weights_match_oracle_pooling():
    N, K = 16 * 37 + 5, 260
    _, W, b = workloads.make_inputs(1, N, K, seed=81)
    Wd, bd = to_dev(W, b)
    with lib.LinEpi() as h:
        Wp, bp = h.pool_weights(Wd, bd, 16)
        torch.cuda.synchronize()
    ref_W = oracle.avgpool1d(W.T.astype(np.float64), 16).T
    ref_b = oracle.avgpool1d(b[None, :].astype(np.float64), 16)[0]
    assert Wp.shape == (37, K) and bp.shape == (37,)
    # 16 fp32 additions then an exact scaling by 1/16: a few ulp
    np.testing.assert_allclose(Wp.cpu().numpy(), ref_W, rtol=0, atol=8 * 2**-24 * np.abs(W).max())
    np.testing.assert_allclose(bp.cpu().numpy(), ref_b, rtol=0, atol=8 * 2**-24 * np.abs(b).max())


def test_pool_weights_worked_example_from_page():
    """Page l2_p98's hand check: x = [1, 2], W = [[1,0],[0,1],[1,1],[2,2]],
    b = 0, window 2 gives pooled weights [[0.5,0.5],[1.5,1.5]] and pooled
    output [1.5, 4.5].  K is padded with zeros to the 4-float row granule."""
    g = json.load(open(os.path.join(GOLDEN, "pool_fold_worked_example.json")))
    pad = lambda a: np.pad(np.array(a, dtype=np.float32), ((0, 0), (0, 2)))
    X, W = pad(g["x"]), pad(g["W"])
    b = np.array(g["b"], dtype=np.float32)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        Wp, bp = h.pool_weights(Wd, bd, g["pool_kernel"])
        y = h.run(Xd, Wp, bp, lib.make_desc(lib.LIN_EPI_NONE))
        torch.cuda.synchronize()
    assert np.array_equal(Wp.cpu().numpy()[:, :2], np.array(g["pooled_weight"], dtype=np.float32))
    assert np.array_equal(y.cpu().numpy(), np.array(g["pooled"], dtype=np.float32))


@pytest.mark.parametrize("M,N,K", [(300, 1024, 520), (37, 6000, 4100), (1, 16, 4), (129, 16 * 33 + 7, 64)])
def test_pool_fold_tail_b_matches_definition(M, N, K):
    """Tail (b) of the original layer, computed as kind 4 on pooled weights,
    against the oracle's unfolded definition (pool the linear output)."""
    X, W, b = workloads.make_inputs(M, N, K, seed=M + 3 * N)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        Wp, bp = h.pool_weights(Wd, bd, 16)
        got = run_gpu(h, Xd, Wp, bp, workloads.TAIL_B_FOLDED)
    compare(got, oracle_rows(X, W, b, workloads.TAIL_B), what="pool-fold %dx%dx%d" % (M, N, K))


def test_pool_fold_full_size_checked_rows():
    w = workloads.WORKLOADS["p2_1024x8192x8192"]
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        Wp, bp = h.pool_weights(Wd, bd, 16)
        got = run_gpu(h, Xd, Wp, bp, workloads.TAIL_B_FOLDED)
        fused = run_gpu(h, Xd, Wd, bd, workloads.TAIL_B)
    rows = workloads.checked_rows(w.M, seed=w.seed)
    ref = oracle_rows(X, W, b, workloads.TAIL_B, rows)
    compare(got[rows], ref, what="pool-fold 1024x8192x8192 (64 rows)")
    # the folded and the direct form agree to fp32 rounding on every row
    compare(got, fused, tol=1e-4, what="pool-fold vs fused direct (all rows)")


# ------------------------------------------------- scale folding, tail (a) (f2)

@pytest.mark.parametrize("M,N,K", [(300, 1040, 520), (1000, 6000, 4100), (64, 256, 256)])
def test_scale_fold_bit_identical_for_power_of_two(M, N, K):
    """Tail (a) on (0.5 W, 0.5 b) with scale 1 equals tail (a) on (W, b) with
    scale 0.5 bit for bit (page l2_p53's pre-scaling idea): scaling by a power
    of two commutes with fp32 rounding.  Both runs use the same plan."""
    X, W, b = workloads.make_inputs(M, N, K, seed=K + 5)
    X *= np.float32(6.0)  # make the clamp fire on part of the outputs
    Xd, Wd, bd = to_dev(X, W, b)
    t = workloads.TAIL_A
    with lib.LinEpi() as h:
        direct = run_gpu(h, Xd, Wd, bd, t)
        Ws, bs = h.scale_weights(Wd, bd, t.scale)
        folded = run_gpu(h, Xd, Ws, bs, workloads.Tail(t.kind, scale=1.0, lo=t.lo, hi=t.hi))
    assert np.array_equal(folded, direct)
    assert np.array_equal(Ws.cpu().numpy(), W * np.float32(0.5))
    compare(folded, oracle_rows(X, W, b, t), what="scale-folded tail a %dx%dx%d" % (M, N, K))


def test_scale_fold_general_scale_within_tolerance():
    X, W, b = workloads.make_inputs(200, 300, 260, seed=3)
    t = workloads.Tail(workloads.SCALE_HARDTANH_GELU, scale=0.3, lo=-1.5, hi=1.0)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        Ws, bs = h.scale_weights(Wd, bd, t.scale)
        folded = run_gpu(h, Xd, Ws, bs, workloads.Tail(t.kind, scale=1.0, lo=t.lo, hi=t.hi))
    compare(folded, oracle_rows(X, W, b, t), what="scale-folded tail a, s=0.3")


# ------------------------------------------------------------- graph capture

@pytest.mark.parametrize("tail", [workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C], ids=lambda t: t.name)
def test_runs_replay_from_a_captured_graph(tail):
    """lin_epi_run enqueues only kernel launches (no memsets, no allocation
    once the workspace exists), so a caller can capture it in a HIP graph.
    One eager run sizes the workspace; the captured graph is then replayed
    several times with other eager work in between, and every replay must
    equal the eager result bit for bit.  Split-K is forced, so every replay
    also relies on the previous one having left the tiles' arrival counters
    at zero."""
    X, W, b = workloads.make_inputs(300, 520, 1040, seed=61)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi(stream=s) as h:
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 3)
        desc = lib.make_desc(tail.kind, tail.scale, tail.lo, tail.hi, tail.pool_kernel)
        Y = torch.empty(lib.LinEpi.output_shape(300, 520, tail.kind), dtype=torch.float32, device="cuda:0")
        with torch.cuda.stream(s):
            h.run_into(Xd, Wd, bd, desc, Y)
        s.synchronize()
        eager = Y.cpu().numpy().copy()
        p = h.plan()
        assert p.split_k == 3 and p.kernels == 1
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            h.run_into(Xd, Wd, bd, desc, Y)
        for i in range(4):
            with torch.cuda.stream(s):
                Y.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
            s.synchronize()
            assert np.array_equal(Y.cpu().numpy(), eager), "replay %d differs" % i
            (Xd[:1] * 2).sum().item()  # unrelated eager work between replays
    compare(eager, oracle_rows(X, W, b, tail), what="graph %s" % tail.name)
