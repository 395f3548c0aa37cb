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
    for code in (-1, -2, -3, -4, -5):
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
    assert lib.lin_epi_set_option(handle, 99, 0) == lib.LIN_EPI_EINVAL
    assert lib.lin_epi_set_option(0, lib.LIN_EPI_OPT_PROFILE, 1) == lib.LIN_EPI_EINVAL
    rc, _ = lib.lin_epi_last_plan(handle)
    assert rc == lib.LIN_EPI_EINVAL  # nothing has run yet
    rc, prof = lib.lin_epi_profile_read(handle)
    assert rc == lib.LIN_EPI_OK and prof.launches[0] == 0 and prof.launches[1] == 0


def test_destroy_null_is_noop():
    assert lib.lin_epi_destroy(0) == lib.LIN_EPI_OK


def test_desc_layout_matches_header():
    assert ctypes.sizeof(lib.lin_epi_desc) == 24
    assert ctypes.sizeof(lib.lin_epi_plan) == 40
    assert ctypes.sizeof(lib.lin_epi_profile) == 32
