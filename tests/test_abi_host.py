"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, and rejects invalid arguments with the
documented status codes before making any HIP call."""

import ctypes
import os
import re

import pytest

import dense_linear_layer_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lin_epi.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lin_epi_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("lin_epi_create", "lin_epi_run", "lin_epi_destroy"):
        assert required in names
    assert sorted(lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    so = lib.load_library()
    for name in _declared_functions():
        assert hasattr(so, name), name
        assert ctypes.cast(getattr(so, name), ctypes.c_void_p).value


def test_status_strings():
    assert lib.lin_epi_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6):
        assert lib.lin_epi_status_string(code) not in ("ok", "unknown status")
    assert lib.lin_epi_status_string(42) == "unknown status"


def test_create_rejects_null_out():
    assert lib.load_library().lin_epi_create(None, None) == lib.LIN_EPI_EINVAL


@pytest.fixture
def handle():
    rc, h = lib.lin_epi_create(None)
    assert rc == lib.LIN_EPI_OK and h
    yield h
    assert lib.lin_epi_destroy(h) == lib.LIN_EPI_OK


# Fake, never dereferenced device addresses: validation must reject every
# call below before any HIP call.
A16 = 0x10000
DESC_A = lib.make_desc(lib.LIN_EPI_SCALE_HARDTANH_GELU, 0.5, -2.0, 2.0)


@pytest.mark.parametrize("args,expect", [
    (dict(h=None), lib.LIN_EPI_EINVAL),
    (dict(desc=None), lib.LIN_EPI_EINVAL),
    (dict(M=-1), lib.LIN_EPI_EINVAL),
    (dict(N=-5), lib.LIN_EPI_EINVAL),
    (dict(K=-4), lib.LIN_EPI_EINVAL),
    (dict(M=2**31), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(7)), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(5)), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(-1)), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(1, 0.5, 2.0, -2.0)), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(2, 2.0, pool_kernel=8)), lib.LIN_EPI_ENOTSUP),
    (dict(desc=lib.make_desc(2, 2.0, pool_kernel=16, pool_stride=8)), lib.LIN_EPI_ENOTSUP),
    (dict(desc=lib.make_desc(2, 2.0), N=15), lib.LIN_EPI_ENOTSUP),
    (dict(b=0), lib.LIN_EPI_EINVAL),
    (dict(Y=0), lib.LIN_EPI_EINVAL),
    (dict(X=0), lib.LIN_EPI_EINVAL),
    (dict(W=0), lib.LIN_EPI_EINVAL),
    (dict(K=6), lib.LIN_EPI_EALIGN),
    (dict(X=A16 + 4), lib.LIN_EPI_EALIGN),
    (dict(W=A16 + 8), lib.LIN_EPI_EALIGN),
    (dict(Y=A16 + 2), lib.LIN_EPI_EALIGN),
    (dict(b=A16 + 1), lib.LIN_EPI_EALIGN),
    # empty problems are successful no-ops, with no device work
    (dict(M=0), lib.LIN_EPI_OK),
    (dict(N=0), lib.LIN_EPI_OK),
    (dict(M=0, X=0, W=0, b=0, Y=0), lib.LIN_EPI_OK),
])
def test_run_validation(handle, args, expect):
    a = dict(h=handle, M=8, N=32, K=16, X=A16, W=A16, b=A16, desc=DESC_A, Y=A16)
    a.update(args)
    rc = lib.lin_epi_run(a["h"], a["M"], a["N"], a["K"], a["X"], a["W"], a["b"], a["desc"], a["Y"])
    assert rc == expect, lib.lin_epi_status_string(rc)


def test_options_and_introspection_validation(handle):
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, -1) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 65) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 3) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_PROFILE, 2) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_UNFUSED, 2) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_UNFUSED, 1) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_UNFUSED, 0) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_REG_STAGING, 2) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_REG_STAGING, 1) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_REG_STAGING, 0) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, -1) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, 2**31) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, 300) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, 0) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, 9) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, -1) == lib.LIN_EPI_EINVAL
    for t in range(8):
        assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, t) == lib.LIN_EPI_OK
    assert lib.lin_epi_set_option(handle, 99, 0) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(0, lib.LIN_EPI_OPT_PROFILE, 1) == lib.LIN_EPI_EINVAL
    rc, _ = lib.lin_epi_last_plan(handle)
    assert rc == lib.LIN_EPI_EINVAL  # nothing has run yet
    rc, prof = lib.lin_epi_profile_read(handle)
    assert rc == lib.LIN_EPI_OK and list(prof.launches) == [0, 0, 0]


@pytest.mark.parametrize("args,expect", [
    (dict(h=None), lib.LIN_EPI_EINVAL),
    (dict(N=-1), lib.LIN_EPI_EINVAL),
    (dict(K=-4), lib.LIN_EPI_EINVAL),
    (dict(pool=0), lib.LIN_EPI_EINVAL),
    (dict(pool=-16), lib.LIN_EPI_EINVAL),
    (dict(b=0), lib.LIN_EPI_EINVAL),
    (dict(bp=0), lib.LIN_EPI_EINVAL),
    (dict(W=0), lib.LIN_EPI_EINVAL),
    (dict(Wp=0), lib.LIN_EPI_EINVAL),
    (dict(K=6), lib.LIN_EPI_EALIGN),
    (dict(W=A16 + 4), lib.LIN_EPI_EALIGN),
    (dict(Wp=A16 + 8), lib.LIN_EPI_EALIGN),
    (dict(bp=A16 + 2), lib.LIN_EPI_EALIGN),
    # fewer rows than one window: nothing to compute
    (dict(N=15), lib.LIN_EPI_OK),
    (dict(N=0, W=0, b=0, Wp=0, bp=0), lib.LIN_EPI_OK),
])
def test_pool_weights_validation(handle, args, expect):
    a = dict(h=handle, N=64, K=16, W=A16, b=A16, pool=16, Wp=A16, bp=A16)
    a.update(args)
    rc = lib.lin_epi_pool_weights(a["h"], a["N"], a["K"], a["W"], a["b"], a["pool"], a["Wp"], a["bp"])
    assert rc == expect, lib.lin_epi_status_string(rc)


@pytest.mark.parametrize("args,expect", [
    (dict(h=None), lib.LIN_EPI_EINVAL),
    (dict(N=-1), lib.LIN_EPI_EINVAL),
    (dict(K=-4), lib.LIN_EPI_EINVAL),
    (dict(b=0), lib.LIN_EPI_EINVAL),
    (dict(bs=0), lib.LIN_EPI_EINVAL),
    (dict(W=0), lib.LIN_EPI_EINVAL),
    (dict(Ws=0), lib.LIN_EPI_EINVAL),
    (dict(K=6), lib.LIN_EPI_EALIGN),
    (dict(W=A16 + 4), lib.LIN_EPI_EALIGN),
    (dict(Ws=A16 + 8), lib.LIN_EPI_EALIGN),
    (dict(b=A16 + 2), lib.LIN_EPI_EALIGN),
    (dict(N=0, W=0, b=0, Ws=0, bs=0), lib.LIN_EPI_OK),
])
def test_scale_weights_validation(handle, args, expect):
    a = dict(h=handle, N=64, K=16, W=A16, b=A16, Ws=A16, bs=A16)
    a.update(args)
    rc = lib.lin_epi_scale_weights(a["h"], a["N"], a["K"], a["W"], a["b"], 0.5, a["Ws"], a["bs"])
    assert rc == expect, lib.lin_epi_status_string(rc)


def test_destroy_null_is_noop():
    assert lib.lin_epi_destroy(0) == lib.LIN_EPI_OK


def test_desc_layout_matches_header():
    assert ctypes.sizeof(lib.lin_epi_desc) == 24
    assert ctypes.sizeof(lib.lin_epi_plan) == 56
    assert ctypes.sizeof(lib.lin_epi_profile) == 48


# ---- the planner, evaluated on the host for a 256-CU device ---------------

def _plan(handle, M, N, K, kind, cus=256):
    rc, p = lib.lin_epi_query_plan(handle, M, N, K, lib.make_desc(kind, 1.0), cus)
    assert rc == lib.LIN_EPI_OK, lib.lin_epi_status_string(rc)
    return (p.tile_m, p.tile_n, p.split_k, p.kernels, p.grid_main, p.workspace_bytes, p.schedule)


def test_planner_choices_for_the_workloads(handle):
    A, B, C, F = (lib.LIN_EPI_SCALE_HARDTANH_GELU, lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX, lib.LIN_EPI_SWISH_SCALE,
                  lib.LIN_EPI_GELU_SCALE_ROWMAX)
    # 2048x8192x8192: 256x256 tiles, one per compute unit, no split, no
    # workspace (128x256 tiles in two rounds measure level with it)
    assert _plan(handle, 2048, 8192, 8192, A) == (256, 256, 1, 1, 256, 0, 0)
    # 128x32768x32768: 128x256 tiles (128 of them) split in two, finished in
    # the GEMM kernel itself (one kernel)
    assert _plan(handle, 128, 32768, 32768, C)[:5] == (128, 256, 2, 1, 256)
    # tail (b) at 1024x8192x8192: whatever the split, the partial sums that
    # reach memory are pooled windows (16x smaller than the raw [M, N] slices,
    # 64 MiB at two slices) plus the per-tile row maxima, which the tile
    # kernel's last workgroup of each tile row reduces (one kernel)
    t = _plan(handle, 1024, 8192, 8192, B)
    assert t[3] == 1 and t[5] < 16 * 2**20, t
    # every elementwise plan is one kernel, with or without split tiles
    t = _plan(handle, 1000, 6000, 4100, A)
    assert t[3] == 1, t
    assert _plan(handle, 128, 32768, 32768, C)[3] == 1
    # few rows against a long weight stream: the weight-streaming kernel
    # (16x64 per wavefront), with at least the 1024 wavefronts that give
    # every SIMD one (256 workgroups of 4)
    for M in (1, 8, 16):
        t = _plan(handle, M, 32768, 32768, C)
        assert t[:2] == (16, 64) and t[4] >= 256, t


def test_planner_page2_never_writes_raw_partials(handle):
    """Tail (b) splits only with pooled partial sums: the workspace holds
    per-tile counters, two slots of (tile / 16) floats per workgroup and the
    per-tile row maxima, never the [M, N] linear output."""
    B = lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX
    for S in (0, 2, 3, 5):
        assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, S) == 0
        tm, tn, s, k, grid, ws, sched = _plan(handle, 1024, 8192, 8192, B)
        tiles = -(-1024 // tm) * -(-8192 // tn)
        slots = grid * (2 if sched == 2 else 1)
        bound = (tiles + -(-1024 // tm)) * 4 + 256 + slots * tm * tn // 16 * 4 + 256 + 1024 * (8192 // tn) * 4 + 256
        assert ws <= bound, (S, ws, bound)
        # raw [M, N] slices would take s * 32 MiB; pooled ones a sixteenth
        assert ws < s * 1024 * 8192 * 4 // 8, (S, ws)
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 0) == 0


def test_planner_grid_option(handle):
    """LIN_EPI_OPT_GRID forces a stream-K grid (clamped to the work), and
    overrides the split option."""
    A = lib.LIN_EPI_SCALE_HARDTANH_GELU
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 3) == 0
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, 300) == 0
    t = _plan(handle, 1000, 6000, 4100, A)
    assert t[4] == 300 and t[6] == 2
    # a grid larger than the (tile, K step) work is clamped to it
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, 4) == 0
    t = _plan(handle, 64, 64, 64, A)
    assert t[4] == 2
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_GRID, 0) == 0
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 0) == 0
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, 0) == 0


def test_planner_respects_options(handle):
    A = lib.LIN_EPI_SCALE_HARDTANH_GELU
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 1) == 0
    assert _plan(handle, 1000, 6000, 4100, A)[2] == 1
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 5) == 0
    assert _plan(handle, 1000, 6000, 4100, A)[2] == 5
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 0) == 0
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_UNFUSED, 1) == 0
    # unfused, no split: GEMM + separate tail kernel; kind 0 has no tail kernel
    assert _plan(handle, 2048, 8192, 8192, A)[3] == 2
    assert _plan(handle, 2048, 8192, 8192, lib.LIN_EPI_NONE)[3] == 1
    # unfused row-max kinds keep the raw output in the workspace
    assert _plan(handle, 2048, 8192, 8192, lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX)[5] >= 2048 * 8192 * 4


def test_planner_tile_override(handle):
    for t, shape in lib.TILE_CONFIGS.items():
        assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, t) == 0
        assert _plan(handle, 2048, 8192, 8192, lib.LIN_EPI_NONE)[:2] == shape
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_TILE, 0) == 0


def test_planner_small_problems_spread_out(handle):
    # 64x256x256 would be one 128x256 workgroup; the planner spreads it over
    # 64x64 tiles and K slices instead
    tm, tn, s, k, grid, _, _ = _plan(handle, 64, 256, 256, lib.LIN_EPI_SCALE_HARDTANH_GELU)
    assert (tm, tn) == (64, 64) and grid >= 4


def test_planner_every_slice_gets_k(handle):
    """For any split the last slice still owns K steps: grid_main = tiles * S and
    S <= ceil(K / 32)."""
    for K in (4, 32, 36, 100, 1000, 4100):
        for S in (2, 3, 5, 16):
            assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, S) == 0
            tm, tn, s, _, grid, _, _ = _plan(handle, 300, 300, K, lib.LIN_EPI_NONE)
            assert 1 <= s <= max(1, -(-K // 32))
            # one workgroup per tile segment; the weight-streaming kernel
            # (16x64) runs four wavefront units per workgroup
            units = -(-300 // tm) * -(-300 // tn) * s
            assert grid == (-(-units // 4) if (tm, tn) == (16, 64) else units)
    assert lib.lin_epi_set_option(handle, lib.LIN_EPI_OPT_SPLIT_K, 0) == 0


def test_query_plan_validation(handle):
    d = lib.make_desc(lib.LIN_EPI_NONE)
    assert lib.lin_epi_query_plan(0, 8, 8, 8, d, 256)[0] == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_query_plan(handle, 8, 8, 8, None, 256)[0] == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_query_plan(handle, 8, 8, 8, d, -1)[0] == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_query_plan(handle, 8, 8, 6, d, 256)[0] == lib.LIN_EPI_EALIGN
    assert lib.lin_epi_query_plan(handle, 8, 8, 8, lib.make_desc(2, pool_kernel=4), 256)[0] == lib.LIN_EPI_ENOTSUP
    rc, p = lib.lin_epi_query_plan(handle, 0, 8, 8, d, 256)
    assert rc == 0 and p.grid_main == 0


# ---- the allocation-free entry point: host-side behaviour ------------------

def test_noalloc_scratch_size():
    assert lib.lin_epi_noalloc_scratch_bytes() == 64 * 2**20


@pytest.mark.parametrize("args,expect", [
    (dict(h=0), lib.LIN_EPI_EINVAL),
    (dict(desc=None), lib.LIN_EPI_EINVAL),
    (dict(M=-1), lib.LIN_EPI_EINVAL),
    (dict(K=6), lib.LIN_EPI_EALIGN),
    (dict(M=0), lib.LIN_EPI_OK),
    (dict(N=0), lib.LIN_EPI_OK),
    (dict(b=0), lib.LIN_EPI_EINVAL),
    (dict(desc=lib.make_desc(2, pool_kernel=8)), lib.LIN_EPI_ENOTSUP),
])
def test_noalloc_validation_before_any_hip_call(handle, args, expect):
    """lin_epi_run_noalloc validates exactly as lin_epi_run does, on the host,
    before touching the device (this container has no GPU)."""
    a = dict(h=handle, M=8, N=32, K=16, X=A16, W=A16, b=A16, desc=DESC_A, Y=A16)
    a.update(args)
    rc = lib.lin_epi_run_noalloc(a["h"], a["M"], a["N"], a["K"], a["X"], a["W"], a["b"], a["desc"], a["Y"])
    assert rc == expect, lib.lin_epi_status_string(rc)


def test_planner_fitted_choices(handle):
    """Plans the fitted time model picks where MI355X timings of every
    candidate plan put them best (or within 1 % of it)."""
    A, B = lib.LIN_EPI_SCALE_HARDTANH_GELU, lib.LIN_EPI_POOL_GELU_SCALE_ROWMAX
    # tail (b) at 1024x8192x8192: 128x256 tiles, one per compute unit, no split
    assert _plan(handle, 1024, 8192, 8192, B)[:5] == (128, 256, 1, 1, 256)
    # the ragged layer, every tail: 64x128 tiles, one per workgroup, 752 of
    # them in one round of three workgroups per compute unit (no partial
    # sums, every workgroup starting at the same K position)
    for kind in (A, B, lib.LIN_EPI_SWISH_SCALE):
        assert _plan(handle, 1000, 6000, 4100, kind)[:5] == (64, 128, 1, 1, 16 * 47)
    # 512x4096x4096: 256 tiles of 64x128, one per compute unit
    assert _plan(handle, 512, 4096, 4096, A)[:5] == (64, 128, 1, 1, 256)
    # 3000x3000x3000: 768 tiles of 128x96 (a round and a half; the 128x256
    # stream-K plan measured 5 % slower)
    assert _plan(handle, 3000, 3000, 3000, A)[:5] == (128, 96, 1, 1, 768)
    # 2000x2000x8192: 512 tiles of 64x128, no split
    assert _plan(handle, 2000, 2000, 8192, A)[:5] == (64, 128, 1, 1, 512)
    # 96 rows: not the 32-row tile (kept for 17-32 rows; at 96 rows it timed
    # 25 % behind the best plan), the 128x96 tile split in two instead
    assert _plan(handle, 96, 12288, 12288, lib.LIN_EPI_SWISH_SCALE)[:5] == (128, 96, 2, 1, 256)
    assert _plan(handle, 32, 16384, 16384, lib.LIN_EPI_SWISH_SCALE)[:2] == (32, 128)
    # 768x3072x3072, 1536x1536x6144, 640x5000x5000: 128x96 stream-K over 256
    # workgroups, one per compute unit (192, 192 and 260 tiles)
    for M, N, K in ((768, 3072, 3072), (1536, 1536, 6144), (640, 5000, 5000)):
        assert _plan(handle, M, N, K, A)[:5] == (128, 96, 2, 1, 256), (M, N, K)


def test_planner_stream_k_stays_within_one_round(handle):
    """Stream-K grids of more than one round of resident workgroups measured
    markedly slower, so the planner never picks one."""
    per_cu = {(256, 256): 1, (128, 256): 1, (128, 128): 2, (64, 64): 4, (32, 128): 4, (64, 128): 3, (128, 96): 2}
    for M, N, K in [(1000, 6000, 4100), (3000, 3000, 3000), (768, 3072, 3072), (300, 530, 1028),
                    (2000, 2000, 8192), (257, 513, 100), (4096, 100, 50000)]:
        for kind in range(5):
            tm, tn, s, k, grid, ws, sched = _plan(handle, M, N, K, kind)
            if sched == 2:
                assert grid <= 256 * per_cu[(tm, tn)], (M, N, K, kind, tm, tn, grid)
