"""The direct-to-LDS staging layout, checked on the CPU for every tile shape
of the library: tests/dma_layout_check.cpp enumerates every DMA instruction,
wavefront and lane of dense_linear_layer_amd/csrc/dma_layout.hpp (the
functions the kernel itself calls) and checks coverage, the swizzle, the
addresses of valid lanes and that every masked lane (row past M or N, chunk
past the K slice) carries a per-lane offset at or beyond num_records."""

import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_linear_layer_amd", "csrc")


def tile_table():
    """(BM, BN, wavefronts) of every TileCfg alias in lin_epi.hip that uses
    the direct-to-LDS path (BK = 32, buffer loads not switched off)."""
    with open(os.path.join(CSRC, "lin_epi.hip")) as f:
        text = f.read()
    shapes = []
    for m in re.finditer(r"using\s+Cfg\w+\s*=\s*TileCfg<([^>]*)>;", text):
        args = [a.strip() for a in m.group(1).split(",")]
        bm, bn, bk, wm, wn = (int(a) for a in args[:5])
        bufload = len(args) < 7 or args[6] == "true"
        if bufload and bk == 32:
            shapes.append((bm, bn, wm * wn))
    return shapes


def test_tile_table_found():
    shapes = tile_table()
    assert (256, 256, 8) in shapes and len(shapes) >= 5, shapes


def test_dma_layout_every_tile(tmp_path):
    shapes = tile_table()
    exe = tmp_path / "dma_layout_check"
    tiles = " ".join("T(%d, %d, %d)" % s for s in shapes)
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__host__=", "-D__device__=", "-DTILES=" + tiles, "-I" + CSRC,
                    os.path.join(ROOT, "tests", "dma_layout_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:]
