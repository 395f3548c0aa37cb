"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
(via the binding), run the CPU oracle on the same seeded inputs, compare."""

from __future__ import annotations

import sys

import numpy as np

import dense_linear_layer_amd as lib
import oracle
import workloads

TOL = 1e-3  # |gpu - ref| <= TOL * (1 + |ref|) on every checked element


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def desc_for(tail: workloads.Tail) -> lib.lin_epi_desc:
    return lib.make_desc(tail.kind, tail.scale, tail.lo, tail.hi, tail.pool_kernel)


def to_dev(*arrays):
    import torch

    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in arrays]


def compare(got: np.ndarray, ref: np.ndarray, tol: float = TOL, what: str = "") -> float:
    """Assert the tolerance on every element; return max |got - ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.isfinite(got).all(), "%s: non-finite GPU output" % what
    err = np.abs(got - ref)
    bad = err > tol * (1.0 + np.abs(ref))
    worst = int(np.argmax(err))
    msg = "%s: max|d|=%.3e at %s (gpu %.9g, ref %.9g); %d/%d outside tolerance" % (
        what, err.flat[worst], np.unravel_index(worst, err.shape), got.flat[worst], ref.flat[worst],
        int(bad.sum()), bad.size)
    log(msg)
    assert not bad.any(), msg
    return float(err.max())


def run_gpu(h: lib.LinEpi, Xd, Wd, bd, tail: workloads.Tail):
    import torch

    Y = h.run(Xd, Wd, bd, desc_for(tail))
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def oracle_rows(X, W, b, tail: workloads.Tail, rows=None):
    return oracle.forward_rows(X, W, b, tail.kind, rows, **tail.params())
