"""The kernel's work partition (dense_linear_layer_amd/csrc/schedule.hpp),
checked on the CPU: tests/schedule_check.cpp replays the kernel's walk over
(tile, K step) iterations for many tile counts, K step counts and grid sizes
(one tile per workgroup, split-K, stream-K) and checks coverage, the segment
bookkeeping the last-arriving workgroup relies on, partial-sum slot
uniqueness, the XCD renumbering, the tile order and the K step grid."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_linear_layer_amd", "csrc")


def test_schedule_partition(tmp_path):
    exe = tmp_path / "schedule_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__host__=", "-D__device__=", "-I" + CSRC,
                    os.path.join(ROOT, "tests", "schedule_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:]
