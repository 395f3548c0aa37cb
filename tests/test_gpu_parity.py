"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, to |gpu - ref| <= 1e-3 * (1 + |ref|) on every checked
element, bit-exact where the exact result is representable."""

import numpy as np
import pytest

import dense_linear_layer_amd as lib
import oracle
import workloads
from parity_util import compare, desc_for, log, oracle_rows, run_gpu, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with lib.LinEpi() as handle:
        yield handle


@pytest.fixture(autouse=True)
def _name(request):
    log("== %s" % request.node.nodeid)


ALL_TAILS = (workloads.TAIL_A, workloads.TAIL_B, workloads.TAIL_C, workloads.TAIL_NONE, workloads.TAIL_B_FOLDED)


# ---------------------------------------------------------------- small shapes

def test_tiny_config_tail_a(h):
    w = workloads.WORKLOADS["tiny"]
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_A)
    compare(got, oracle_rows(X, W, b, workloads.TAIL_A), what="tiny tail a")


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (37, 200, 68), (129, 130, 36), (1, 1, 4), (7, 33, 4),
                                   (300, 17, 1028), (1000, 6000, 4100)])
def test_integer_inputs_bit_exact(h, M, N, K):
    """Integer-valued inputs: every partial sum is an exact fp32 integer, so the
    GPU must reproduce the oracle bit for bit whatever its summation order.
    Pins indexing, K tail and edge masking."""
    X, W, b = workloads.integer_inputs(M, N, K, seed=M + N + K)
    got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
    ref = oracle.linear_rows(X, W, b)
    assert np.array_equal(got.astype(np.float64), ref), "max|d| = %g" % np.abs(got - ref).max()


@pytest.mark.parametrize("M,N,K", [(5, 48, 12), (130, 290, 100), (257, 64, 520), (64, 16, 8), (33, 1000, 4)])
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_odd_shapes_all_tails(h, M, N, K, tail):
    X, W, b = workloads.make_inputs(M, N, K, seed=3 * M + N)
    got = run_gpu(h, *to_dev(X, W, b), tail)
    compare(got, oracle_rows(X, W, b, tail), what="%dx%dx%d %s" % (M, N, K, tail.name))


def test_ragged_config_all_tails_on_one_gemm(h):
    """1000x6000x4100: not tile multiples; the three tails run on the same X, W, b
    (tail (b) pools 6000 columns into 375 windows)."""
    w = workloads.WORKLOADS["ragged_1000x6000x4100"]
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    Xd, Wd, bd = to_dev(X, W, b)
    y = oracle.linear_rows(X, W, b)
    for tail in w.tails:
        got = run_gpu(h, Xd, Wd, bd, tail)
        ref = oracle.apply_tail(y, tail.kind, **tail.params())
        compare(got, ref, what="ragged %s" % tail.name)
        if tail.kind == workloads.POOL_GELU_SCALE_ROWMAX:
            _, g, _ = oracle.tail_pool_gelu_scale_rowmax(y, 16, tail.scale)
            assert g.shape[1] == 375


def test_k_zero_gives_tail_of_bias(h):
    M, N = 70, 300
    b = workloads.make_inputs(1, N, 4, seed=11)[2]
    X = torch.empty((M, 0), dtype=torch.float32, device="cuda:0")
    W = torch.empty((N, 0), dtype=torch.float32, device="cuda:0")
    bd = to_dev(b)[0]
    for tail in ALL_TAILS:
        got = run_gpu(h, X, W, bd, tail)
        ref = oracle.apply_tail(np.tile(b.astype(np.float64), (M, 1)), tail.kind, **tail.params())
        compare(got, ref, what="K=0 %s" % tail.name)


# ------------------------------------------------- epilogue functors, tightly

def _functor_inputs(n_values: int):
    """X = I_K and b = 0 make the GEMM exact: Y[m, n] = W[n, m].  W carries a
    dense grid of values in [-10, 10] plus the clamp points and their
    neighbours, so Y = tail(W^T) exposes the epilogue math alone."""
    vals = np.linspace(-10, 10, n_values - 12).astype(np.float32)
    extra = np.array([0.0, -0.0, 2.0, -2.0, 4.0, -4.0, np.nextafter(np.float32(4), np.float32(5)),
                      np.nextafter(np.float32(4), np.float32(3)), np.nextafter(np.float32(-4), np.float32(-5)),
                      np.nextafter(np.float32(-4), np.float32(-3)), 1.0, -1.0], dtype=np.float32)
    vals = np.concatenate([vals, extra])
    K = 128
    N = vals.size // K
    W = vals[: N * K].reshape(N, K).copy()
    X = np.eye(K, dtype=np.float32)
    b = np.zeros(N, dtype=np.float32)
    return X, W, b


@pytest.mark.parametrize("tail", [workloads.TAIL_A, workloads.TAIL_C, workloads.TAIL_NONE], ids=lambda t: t.name)
def test_epilogue_functor_accuracy(h, tail):
    X, W, b = _functor_inputs(128 * 96)
    got = run_gpu(h, *to_dev(X, W, b), tail)
    ref = oracle_rows(X, W, b, tail)
    err = np.abs(got.astype(np.float64) - ref)
    rel = (err / (1.0 + np.abs(ref))).max()
    log("functor %s max|d| = %.3g, max|d|/(1+|ref|) = %.3g" % (tail.name, err.max(), rel))
    # a few fp32 ulp of the output; erf-GELU and tanh-GELU differ by up to 4.7e-4
    assert rel <= 2e-6


def test_tail_a_clipping_exercised(h):
    """X scaled by 10 so that about half of y*0.5 lies outside [-2, 2]."""
    X, W, b = workloads.make_inputs(300, 520, 256, seed=21)
    X *= np.float32(10.0)
    y = oracle.linear_rows(X, W, b)
    frac = float((np.abs(0.5 * y) > 2).mean())
    assert frac > 0.3
    got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_A)
    compare(got, oracle.apply_tail(y, workloads.SCALE_HARDTANH_GELU, **workloads.TAIL_A.params()),
            what="clipping tail a (%.0f%% clipped)" % (100 * frac))


# ------------------------------------------------------------------ split-K

@pytest.mark.parametrize("S", [2, 3, 5])
@pytest.mark.parametrize("tail", [workloads.TAIL_A, workloads.TAIL_C, workloads.TAIL_NONE, workloads.TAIL_B,
                                  workloads.TAIL_B_FOLDED], ids=lambda t: t.name)
def test_forced_split_k(tail, S):
    M, N, K = 200, 390, 1000
    X, W, b = workloads.make_inputs(M, N, K, seed=31)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, S)
        Xd, Wd, bd = to_dev(X, W, b)
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        # the last workgroup of each tile adds the K segments, and for the
        # row-max tails the last of each tile row takes the row maximum, in
        # the GEMM kernel itself
        assert p.split_k == S and p.schedule == 1
        assert p.kernels == 1
        compare(got, oracle_rows(X, W, b, tail), what="split-K %d %s" % (S, tail.name))
        again = [run_gpu(h, Xd, Wd, bd, tail) for _ in range(2)]
        for a in again:
            assert np.array_equal(a, got), "split-K rerun not bitwise identical"


def test_split_k_integer_exact():
    X, W, b = workloads.integer_inputs(130, 260, 2052, seed=32)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 4)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
        assert h.plan().split_k == 4
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))


# ------------------------------------------------------------- determinism

def test_rowmax_deterministic(h):
    X, W, b = workloads.make_inputs(500, 3000, 520, seed=41)
    Xd, Wd, bd = to_dev(X, W, b)
    outs = [run_gpu(h, Xd, Wd, bd, workloads.TAIL_B) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    compare(outs[0], oracle_rows(X, W, b, workloads.TAIL_B), what="rowmax 500x3000x520")


# ---------------------------------------------------------------- guard bands

@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_output_guard_bands_untouched(h, tail):
    M, N, K = 131, 200, 36
    X, W, b = workloads.make_inputs(M, N, K, seed=51)
    Xd, Wd, bd = to_dev(X, W, b)
    n_out = int(np.prod(lib.LinEpi.output_shape(M, N, tail.kind)))
    pad = 4096
    buf = torch.full((n_out + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda:0")
    Y = buf[pad: pad + n_out]
    h.run_into(Xd, Wd, bd, desc_for(tail), Y)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.isnan(host[:pad]).all() and np.isnan(host[pad + n_out:]).all(), "write outside Y"
    ref = oracle_rows(X, W, b, tail)
    compare(host[pad: pad + n_out].reshape(ref.shape), ref, what="guarded %s" % tail.name)


def test_non_default_stream():
    X, W, b = workloads.make_inputs(260, 300, 64, seed=61)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi(stream=s) as h:
        with torch.cuda.stream(s):
            Y = h.run(Xd, Wd, bd, desc_for(workloads.TAIL_C))
        s.synchronize()
        compare(Y.cpu().numpy(), oracle_rows(X, W, b, workloads.TAIL_C), what="side stream")


def test_bound_stream_called_from_another_stream():
    """A handle bound to a side stream, called while torch's current stream is
    the default one: Y is allocated on the handle's stream and the inputs are
    marked as used there, so freeing them right after the call is safe."""
    X, W, b = workloads.make_inputs(260, 300, 64, seed=62)
    s = torch.cuda.Stream()
    Xd, Wd, bd = to_dev(X, W, b)
    torch.cuda.synchronize()
    with lib.LinEpi(stream=s) as h:
        Y = h.run(Xd, Wd, bd, desc_for(workloads.TAIL_A))
        del Xd, Wd, bd  # the allocator must not reuse these before s has finished
        junk = [torch.full((260 * 64,), float("nan"), device="cuda:0") for _ in range(4)]
        s.synchronize()
        del junk
        compare(Y.cpu().numpy(), oracle_rows(X, W, b, workloads.TAIL_A), what="bound stream, other current stream")


# ------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["p1_2048x8192x8192", "p2_1024x8192x8192", "p3_128x32768x32768",
                                  "p3_m16_16x32768x32768", "p3_m8_8x32768x32768", "p3_m1_1x32768x32768"])
def test_full_size_workload_checked_rows(h, name):
    """The large shapes at full size, in the launch configuration the benchmark
    times, checked on 64 seeded rows (all N outputs of each row)."""
    w = workloads.WORKLOADS[name]
    log("generating %s" % name)
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    Xd, Wd, bd = to_dev(X, W, b)
    rows = workloads.checked_rows(w.M, seed=w.seed)
    tail = w.tails[0]
    log("running %s on the GPU (plan follows)" % name)
    got = run_gpu(h, Xd, Wd, bd, tail)
    p = h.plan()
    log("plan: tile %dx%dx%d split %d grid %d kernels %d" % (p.tile_m, p.tile_n, p.tile_k, p.split_k, p.grid_main,
                                                            p.kernels))
    del Wd
    torch.cuda.empty_cache()
    log("oracle on %d rows" % rows.size)
    ref = oracle_rows(X, W, b, tail, rows)
    compare(got[rows], ref, what="%s %s (64 rows)" % (name, tail.name))


@pytest.mark.parametrize("tail", [workloads.TAIL_A, workloads.TAIL_C, workloads.TAIL_B], ids=lambda t: t.name)
def test_split_k_output_offset_by_one_float(tail):
    """Y starting 4 bytes past a 16-byte boundary with split tiles: the
    workgroup that finishes each tile writes exactly Y, nothing around it."""
    M, N, K = 70, 264, 1000
    X, W, b = workloads.make_inputs(M, N, K, seed=91)
    Xd, Wd, bd = to_dev(X, W, b)
    n_out = int(np.prod(lib.LinEpi.output_shape(M, N, tail.kind)))
    buf = torch.full((n_out + 8,), float("nan"), dtype=torch.float32, device="cuda:0")
    Y = buf[1: 1 + n_out]
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 3)
        h.run_into(Xd, Wd, bd, desc_for(tail), Y)
        torch.cuda.synchronize()
        assert h.plan().split_k == 3
    host = buf.cpu().numpy()
    assert np.isnan(host[0]) and np.isnan(host[1 + n_out:]).all()
    ref = oracle_rows(X, W, b, tail)
    compare(host[1: 1 + n_out].reshape(ref.shape), ref, what="offset Y split-3 %s" % tail.name)


# ------------------------------------------------- every tile configuration

@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("tile", sorted(lib.TILE_CONFIGS))
@pytest.mark.parametrize("M,N,K", [(37, 200, 68), (300, 17, 1028), (257, 513, 100), (1, 1, 4)])
def test_every_tile_config_integer_exact(tile, split, M, N, K):
    """The planner may pick any configuration; each one must be bit-exact on
    integer inputs, with and without split-K, on shapes ragged in M, N, K."""
    X, W, b = workloads.integer_inputs(M, N, K, seed=M * N + K)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
        p = h.plan()
        assert (p.tile_m, p.tile_n) == lib.TILE_CONFIGS[tile]
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))


@pytest.mark.parametrize("tile", sorted(lib.TILE_CONFIGS))
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_every_tile_config_all_tails(tile, tail):
    M, N, K = 130, 290, 100
    X, W, b = workloads.make_inputs(M, N, K, seed=tile)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 1)
        got = run_gpu(h, *to_dev(X, W, b), tail)
    compare(got, oracle_rows(X, W, b, tail), what="tile %d %s" % (tile, tail.name))


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("tile", sorted(lib.TILE_CONFIGS))
@pytest.mark.parametrize("tail", ALL_TAILS, ids=lambda t: t.name)
def test_direct_to_lds_equals_register_staging(tile, split, tail):
    """Every tile stages operands with direct-to-LDS buffer loads into a
    swizzled layout by default; forced register staging (padded rows) must
    give bit-identical results on random inputs, ragged in M, N and K, since
    both feed the same MFMA sequence.  Also checked against the oracle."""
    M, N, K = 261, 530, 1000
    X, W, b = workloads.make_inputs(M, N, K, seed=100 * tile + split)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, tile)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        direct = run_gpu(h, Xd, Wd, bd, tail)
        h.set_option(lib.LIN_EPI_OPT_REG_STAGING, 1)
        staged = run_gpu(h, Xd, Wd, bd, tail)
        assert h.plan().split_k == split
    assert np.array_equal(direct, staged), "staging paths differ (tile %d split %d %s)" % (tile, split, tail.name)
    compare(direct, oracle_rows(X, W, b, tail), what="tile %d split %d %s" % (tile, split, tail.name))


# ------------------------------------------------------------- maximum sizes

@pytest.mark.parametrize("tail", [workloads.TAIL_C, workloads.TAIL_B], ids=lambda t: t.name)
def test_output_beyond_2_to_31_elements(tail):
    """M x N above 2^31 (an 8.6 GB output for the elementwise tail): every
    output offset beyond 32 bits must land where the oracle says.  Rows are
    sampled on the device (the output is never copied whole)."""
    M, N, K = 65536 + 37, 32768, 68
    assert M * N > 2**31
    X, W, b = workloads.make_inputs(M, N, K, seed=77)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        Y = h.run(Xd, Wd, bd, desc_for(tail))
        torch.cuda.synchronize()
        p = h.plan()
        log("plan: tile %dx%d split %d grid %d" % (p.tile_m, p.tile_n, p.split_k, p.grid_main))
    rows = np.array([0, 1, 65535, 65536, M - 2, M - 1, 40000, 12345])
    got = Y[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    del Y
    torch.cuda.empty_cache()
    compare(got, oracle_rows(X, W, b, tail, rows), what="M*N > 2^31, %s" % tail.name)


def test_row_max_partials_beyond_2_gib_per_tile_row():
    """Tail (b) on 256x256 tiles with 2^21 + 1 column tiles: one tile row's
    per-tile row maxima (256 rows x 2^21 + 1 tiles x 4 bytes) span more than
    2^31 bytes, so the tile kernel's partial stores and its last workgroup's
    read-back must use 64-bit offsets.  W is 8.6 GB (K = 4)."""
    M, N, K = 257, 2**29 + 48, 4
    tail = workloads.TAIL_B
    assert 256 * -(-N // 256) * 4 > 2**31
    X, W, b = workloads.make_inputs(M, N, K, seed=29)
    Xd, Wd, bd = to_dev(X, W, b)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, 1)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, 1)
        got = run_gpu(h, Xd, Wd, bd, tail)
        p = h.plan()
        assert (p.tile_m, p.tile_n, p.kernels) == (256, 256, 1)
    del Xd, Wd, bd
    torch.cuda.empty_cache()
    # row 255's partials of the last column tiles lie past byte 2^31
    rows = np.array([0, 255, 256])
    compare(got[rows], oracle_rows(X, W, b, tail, rows), what="row-max partials > 2 GiB per tile row")


@pytest.mark.parametrize("K", [2**20 - 4, 2**20])
@pytest.mark.parametrize("split", [1, 3])
def test_long_k_across_the_buffer_window(K, split):
    """With 256-row tiles, K = 2^20 is the first length whose tile rows span
    the buffer-load window (rows * K * 4 bytes = 2^30), so the kernel falls
    back to predicated loads; K = 2^20 - 4 is the last that uses buffer loads.
    Integer inputs keep every sum exact (|sum| <= 4 K < 2^24)."""
    M, N = 3, 37
    X, W, b = workloads.integer_inputs(M, N, K, seed=K % 1000 + split)
    with lib.LinEpi() as h:
        h.set_option(lib.LIN_EPI_OPT_TILE, 1)
        h.set_option(lib.LIN_EPI_OPT_SPLIT_K, split)
        got = run_gpu(h, *to_dev(X, W, b), workloads.TAIL_NONE)
    assert np.array_equal(got.astype(np.float64), oracle.linear_rows(X, W, b))
