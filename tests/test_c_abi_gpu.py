"""The C ABI end to end from plain C on the GPU: tests/c_abi_gpu.c (built by
__graft_entry__.build() as tests/c_abi_gpu.bin) allocates device buffers with
the HIP runtime, calls lin_epi_run on the default stream and on a stream of
its own, and checks the results against the CPU oracle: integer inputs
bit-exact, tails (a) and (b) within 1e-3 * (1 + |ref|)."""

import os
import subprocess

import pytest

from parity_util import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_gpu.bin")


def test_c_program_runs_the_hot_path_on_the_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # build() always produces the binary, so its absence is a failure, not a skip
    assert os.path.exists(BIN), "tests/c_abi_gpu.bin is not built (python -c 'import __graft_entry__ as g; g.build()')"
    log("== running %s" % BIN)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), out
