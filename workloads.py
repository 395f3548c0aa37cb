"""Seeded synthetic workloads for the fused linear layer.

This module only draws inputs and names the shapes; it holds none of the
layer's arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle
consume the arrays it returns, so the two sides always see identical inputs.

Initialisation follows nn.Linear's default, which page "Kimi-K2.6 l2_p53"
(its ModelNew construction) and page "Kimi-K2.6 l2_p98" (its numerics
discussion, corrected to Kaiming-uniform bounds) describe: weights and bias
uniform in (-1/sqrt(in_features), +1/sqrt(in_features)).  Inputs are standard
normal.  The pages do not evaluate on any dataset; these draws stand in for
the benchmark problems' ``get_inputs``.

Recipe (numpy PCG64, ``numpy.random.default_rng(seed)``), drawn in this order,
all float32:

    X = rng.standard_normal((M, K), dtype=float32)
    W = (rng.random((N, K), dtype=float32) * 2 - 1) * TK     (in row chunks)
    b = (rng.random(N, dtype=float32) * 2 - 1) * TK

with ``TK = float32(1 / sqrt(K))``.  Checked rows for the large shapes are
{0, M-1} plus 62 distinct rows from ``default_rng(seed + 1)``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Tail kinds (the numbering of the C interface's epilogue descriptor).
NONE, SCALE_HARDTANH_GELU, POOL_GELU_SCALE_ROWMAX, SWISH_SCALE, GELU_SCALE_ROWMAX = 0, 1, 2, 3, 4

TAIL_NAMES = {
    NONE: "linear",
    SCALE_HARDTANH_GELU: "scale_hardtanh_gelu",
    POOL_GELU_SCALE_ROWMAX: "avgpool16_gelu_scale_rowmax",
    SWISH_SCALE: "swish_scale",
    GELU_SCALE_ROWMAX: "gelu_scale_rowmax",
}


@dataclass(frozen=True)
class Tail:
    kind: int
    scale: float = 1.0
    lo: float = -1.0
    hi: float = 1.0
    pool_kernel: int = 16

    def params(self) -> dict:
        return dict(scale=self.scale, lo=self.lo, hi=self.hi, pool_kernel=self.pool_kernel)

    @property
    def name(self) -> str:
        return TAIL_NAMES[self.kind]


TAIL_A = Tail(SCALE_HARDTANH_GELU, scale=0.5, lo=-2.0, hi=2.0)   # page l2_p53
TAIL_B = Tail(POOL_GELU_SCALE_ROWMAX, scale=2.0, pool_kernel=16)  # page l2_p98
TAIL_C = Tail(SWISH_SCALE, scale=2.0)                             # page l2_p59
TAIL_NONE = Tail(NONE)
TAIL_B_FOLDED = Tail(GELU_SCALE_ROWMAX, scale=2.0)                # tail (b) on pooled weights


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    tails: tuple = field(default_factory=tuple)
    seed: int = 0
    bound: str = "mfma"  # the roofline that bounds it: "mfma" or "hbm"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self, tail: Tail) -> int:
        """Compulsory HBM bytes of one call: X, W, b read once, Y written once."""
        out = self.M if tail.kind in (POOL_GELU_SCALE_ROWMAX, GELU_SCALE_ROWMAX) else self.M * self.N
        return 4 * (self.M * self.K + self.N * self.K + self.N + out)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 256, (TAIL_A,)),
    "p1_2048x8192x8192": Workload("p1_2048x8192x8192", 2048, 8192, 8192, (TAIL_A,)),
    "p2_1024x8192x8192": Workload("p2_1024x8192x8192", 1024, 8192, 8192, (TAIL_B,)),
    "p3_128x32768x32768": Workload("p3_128x32768x32768", 128, 32768, 32768, (TAIL_C,)),
    "ragged_1000x6000x4100": Workload("ragged_1000x6000x4100", 1000, 6000, 4100, (TAIL_A, TAIL_B, TAIL_C)),
    # page l2_p59's layer with decode-size batches: 16, 8 and 1 rows against
    # a 4 GiB weight, bounded by streaming W from HBM rather than by the
    # matrix cores
    "p3_m16_16x32768x32768": Workload("p3_m16_16x32768x32768", 16, 32768, 32768, (TAIL_C,), bound="hbm"),
    "p3_m8_8x32768x32768": Workload("p3_m8_8x32768x32768", 8, 32768, 32768, (TAIL_C,), bound="hbm"),
    "p3_m1_1x32768x32768": Workload("p3_m1_1x32768x32768", 1, 32768, 32768, (TAIL_C,), bound="hbm"),
    # not one of the pages' layers: a square shape whose tiles do not fill
    # whole rounds, where the planner picks the 128x96 tile (timed for it)
    "square_3000x3000x3000": Workload("square_3000x3000x3000", 3000, 3000, 3000, (TAIL_A,)),
}


def bound(K: int) -> np.float32:
    """Kaiming-uniform bound 1/sqrt(fan_in) as float32 (1.0 for K == 0)."""
    return np.float32(1.0 / np.sqrt(K)) if K > 0 else np.float32(1.0)


def make_inputs(M: int, N: int, K: int, seed: int = 0, chunk_rows: int = 4096):
    """Draw X [M,K], W [N,K], b [N] (float32, C-contiguous) per the module recipe."""
    rng = np.random.default_rng(seed)
    tk = bound(K)
    X = rng.standard_normal((M, K), dtype=np.float32)
    W = np.empty((N, K), dtype=np.float32)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        u = rng.random((r1 - r0, K), dtype=np.float32)
        u *= np.float32(2.0)
        u -= np.float32(1.0)
        u *= tk
        W[r0:r1] = u
    b = rng.random(N, dtype=np.float32)
    b *= np.float32(2.0)
    b -= np.float32(1.0)
    b *= tk
    return X, W, b


def checked_rows(M: int, seed: int = 0, count: int = 64) -> np.ndarray:
    """Rows compared against the oracle for large shapes: {0, M-1} plus
    ``count - 2`` distinct others drawn with default_rng(seed + 1); all rows
    when M <= count."""
    if M <= count:
        return np.arange(M, dtype=np.int64)
    rng = np.random.default_rng(seed + 1)
    inner = rng.choice(np.arange(1, M - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], inner]).astype(np.int64))


def integer_inputs(M: int, N: int, K: int, seed: int = 0, lo: int = -2, hi: int = 2):
    """Integer-valued float32 X, W, b with entries in [lo, hi].  For K * hi^2
    below 2^24 every partial sum is an exactly representable integer, so any
    fp32 summation order gives the exact result."""
    rng = np.random.default_rng(seed)
    X = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    W = rng.integers(lo, hi + 1, size=(N, K)).astype(np.float32)
    b = rng.integers(lo, hi + 1, size=N).astype(np.float32)
    return X, W, b
