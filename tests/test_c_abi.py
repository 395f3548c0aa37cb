"""The C ABI from plain C: compile tests/c_abi_check.c with gcc as C99
(-Wall -Wextra -Werror -pedantic) against include/lin_epi.h, link the built
library, run it.  Host-side paths only; no GPU needed.  A second build adds
AddressSanitizer and UndefinedBehaviorSanitizer to the C program."""

import os
import subprocess

import pytest

import dense_linear_layer_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_check.c")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(lib.LIB_PATH)


def _build_and_run(tmp_path, extra):
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", *extra, "-I" + INCLUDE, SRC,
           "-L" + LIBDIR, "-llin_epi", "-Wl,-rpath," + LIBDIR, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    return r.returncode, r.stdout + r.stderr


def test_header_compiles_as_c99_and_abi_runs(tmp_path):
    lib.load_library()  # fails loudly if the library is not built
    rc, out = _build_and_run(tmp_path, ["-O1"])
    assert rc == 0 and out.strip().endswith("ok"), out


def test_c_caller_under_sanitizers(tmp_path):
    probe = subprocess.run(["gcc", "-fsanitize=address,undefined", "-x", "c", "-", "-o", str(tmp_path / "p")],
                           input="int main(void){return 0;}", capture_output=True, text=True)
    if probe.returncode != 0:
        pytest.skip("gcc sanitizers unavailable")
    rc, out = _build_and_run(tmp_path, ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"])
    assert rc == 0 and out.strip().endswith("ok"), out


def test_library_host_code_under_sanitizers(tmp_path):
    """The library itself with AddressSanitizer + UndefinedBehaviorSanitizer on
    its host code (device code is untouched: the flags go to the host pass
    only), driven by the same C program built with clang, leak checking on."""
    hipcc = "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    so = str(tmp_path / "liblin_epi.so")
    csrc = os.path.join(ROOT, "dense_linear_layer_amd", "csrc")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-I" + INCLUDE, "-I" + csrc, os.path.join(csrc, "lin_epi.hip"), "-o", so],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "c_abi_check_san")
    subprocess.run([clang, "-std=c99", "-Wall", "-Werror", "-O1", "-g", "-fsanitize=address,undefined",
                    "-I" + INCLUDE, SRC, "-L" + str(tmp_path), "-llin_epi", "-Wl,-rpath," + str(tmp_path), "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
