"""Python binding of the fused fp32 linear layer library (liblin_epi.so).

The functions below carry the C names of ``include/lin_epi.h`` and only
marshal arguments (ctypes); every step of the computation runs in the HIP
kernels of the library.  PyTorch is used for device memory and streams only,
in :class:`LinEpi`.  There is no CPU fallback: if the library is missing, the
first call raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblin_epi.so")

# lin_epi_kind
LIN_EPI_NONE = 0
LIN_EPI_SCALE_HARDTANH_GELU = 1
LIN_EPI_POOL_GELU_SCALE_ROWMAX = 2
LIN_EPI_SWISH_SCALE = 3
LIN_EPI_GELU_SCALE_ROWMAX = 4

# status codes
LIN_EPI_OK = 0
LIN_EPI_EINVAL = -1
LIN_EPI_EALIGN = -2
LIN_EPI_ENOTSUP = -3
LIN_EPI_ENOMEM = -4
LIN_EPI_EHIP = -5
LIN_EPI_ETOOBIG = -6

# options
LIN_EPI_OPT_SPLIT_K = 1
LIN_EPI_OPT_PROFILE = 2
LIN_EPI_OPT_UNFUSED = 3
LIN_EPI_OPT_TILE = 4
LIN_EPI_OPT_REG_STAGING = 5
LIN_EPI_OPT_GRID = 6
# tile option -> (tile_m, tile_n) the plan reports; 6 is the weight-streaming
# kernel (16 rows of X against 64 rows of W per wavefront)
TILE_CONFIGS = {1: (256, 256), 2: (128, 256), 3: (128, 128), 4: (64, 64), 5: (32, 128), 6: (16, 64), 7: (64, 128), 8: (128, 96)}
TILE_DECODE = 6  # its K segments come from LIN_EPI_OPT_SPLIT_K; it has no stream-K grid

# every function include/lin_epi.h declares
EXPORTS = (
    "lin_epi_create",
    "lin_epi_run",
    "lin_epi_run_noalloc",
    "lin_epi_noalloc_scratch_bytes",
    "lin_epi_destroy",
    "lin_epi_status_string",
    "lin_epi_pool_weights",
    "lin_epi_scale_weights",
    "lin_epi_set_option",
    "lin_epi_last_plan",
    "lin_epi_query_plan",
    "lin_epi_profile_read",
)


class lin_epi_desc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("ht_min", ctypes.c_float),
        ("ht_max", ctypes.c_float),
        ("pool_kernel", ctypes.c_int32),
        ("pool_stride", ctypes.c_int32),
    ]


class lin_epi_plan(ctypes.Structure):
    _fields_ = [
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("tile_k", ctypes.c_int32),
        ("split_k", ctypes.c_int32),
        ("grid_main", ctypes.c_int64),
        ("kernels", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("schedule", ctypes.c_int32),
        ("partial_bytes", ctypes.c_int64),
    ]


class lin_epi_profile(ctypes.Structure):
    _fields_ = [
        ("launches", ctypes.c_int64 * 3),
        ("total_ms", ctypes.c_double * 3),
    ]


class LinEpiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, lin_epi_status_string(status), status))


_lib = None


def load_library():
    """Load liblin_epi.so (built in-tree by dense_linear_layer_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("liblin_epi.so is not built (%s); run `python -m dense_linear_layer_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.lin_epi_create.argtypes = [ctypes.POINTER(p), p]
    lib.lin_epi_create.restype = ctypes.c_int
    lib.lin_epi_run.argtypes = [p, i64, i64, i64, p, p, p, ctypes.POINTER(lin_epi_desc), p]
    lib.lin_epi_run.restype = ctypes.c_int
    lib.lin_epi_run_noalloc.argtypes = [p, i64, i64, i64, p, p, p, ctypes.POINTER(lin_epi_desc), p]
    lib.lin_epi_run_noalloc.restype = ctypes.c_int
    lib.lin_epi_noalloc_scratch_bytes.argtypes = []
    lib.lin_epi_noalloc_scratch_bytes.restype = i64
    lib.lin_epi_destroy.argtypes = [p]
    lib.lin_epi_destroy.restype = ctypes.c_int
    lib.lin_epi_status_string.argtypes = [ctypes.c_int]
    lib.lin_epi_status_string.restype = ctypes.c_char_p
    lib.lin_epi_pool_weights.argtypes = [p, i64, i64, p, p, i32, p, p]
    lib.lin_epi_pool_weights.restype = ctypes.c_int
    lib.lin_epi_scale_weights.argtypes = [p, i64, i64, p, p, ctypes.c_float, p, p]
    lib.lin_epi_scale_weights.restype = ctypes.c_int
    lib.lin_epi_set_option.argtypes = [p, i32, i64]
    lib.lin_epi_set_option.restype = ctypes.c_int
    lib.lin_epi_last_plan.argtypes = [p, ctypes.POINTER(lin_epi_plan)]
    lib.lin_epi_last_plan.restype = ctypes.c_int
    lib.lin_epi_query_plan.argtypes = [p, i64, i64, i64, ctypes.POINTER(lin_epi_desc), i32,
                                       ctypes.POINTER(lin_epi_plan)]
    lib.lin_epi_query_plan.restype = ctypes.c_int
    lib.lin_epi_profile_read.argtypes = [p, ctypes.POINTER(lin_epi_profile)]
    lib.lin_epi_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


# ---- the C entry points, same names, plain integers for pointers ----------

def lin_epi_status_string(status: int) -> str:
    return load_library().lin_epi_status_string(int(status)).decode()


def lin_epi_create(hip_stream: int | None = None) -> tuple[int, int]:
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    rc = load_library().lin_epi_create(ctypes.byref(h), ctypes.c_void_p(hip_stream or None))
    return rc, (h.value or 0)


def lin_epi_run(handle: int, M: int, N: int, K: int, X: int, W: int, b: int, desc: lin_epi_desc | None,
                Y: int) -> int:
    d = ctypes.byref(desc) if desc is not None else None
    return load_library().lin_epi_run(ctypes.c_void_p(handle or None), M, N, K, ctypes.c_void_p(X or None),
                                      ctypes.c_void_p(W or None), ctypes.c_void_p(b or None), d,
                                      ctypes.c_void_p(Y or None))


def lin_epi_run_noalloc(handle: int, M: int, N: int, K: int, X: int, W: int, b: int, desc: lin_epi_desc | None,
                        Y: int) -> int:
    d = ctypes.byref(desc) if desc is not None else None
    return load_library().lin_epi_run_noalloc(ctypes.c_void_p(handle or None), M, N, K, ctypes.c_void_p(X or None),
                                              ctypes.c_void_p(W or None), ctypes.c_void_p(b or None), d,
                                              ctypes.c_void_p(Y or None))


def lin_epi_noalloc_scratch_bytes() -> int:
    return int(load_library().lin_epi_noalloc_scratch_bytes())


def lin_epi_destroy(handle: int) -> int:
    return load_library().lin_epi_destroy(ctypes.c_void_p(handle or None))


def lin_epi_pool_weights(handle: int, N: int, K: int, W: int, b: int, pool_kernel: int, Wp: int, bp: int) -> int:
    return load_library().lin_epi_pool_weights(ctypes.c_void_p(handle or None), N, K, ctypes.c_void_p(W or None),
                                               ctypes.c_void_p(b or None), pool_kernel, ctypes.c_void_p(Wp or None),
                                               ctypes.c_void_p(bp or None))


def lin_epi_scale_weights(handle: int, N: int, K: int, W: int, b: int, scale: float, Ws: int, bs: int) -> int:
    return load_library().lin_epi_scale_weights(ctypes.c_void_p(handle or None), N, K, ctypes.c_void_p(W or None),
                                                ctypes.c_void_p(b or None), float(scale), ctypes.c_void_p(Ws or None),
                                                ctypes.c_void_p(bs or None))


def lin_epi_set_option(handle: int, option: int, value: int) -> int:
    return load_library().lin_epi_set_option(ctypes.c_void_p(handle or None), option, value)


def lin_epi_last_plan(handle: int) -> tuple[int, lin_epi_plan]:
    p = lin_epi_plan()
    rc = load_library().lin_epi_last_plan(ctypes.c_void_p(handle or None), ctypes.byref(p))
    return rc, p


def lin_epi_query_plan(handle: int, M: int, N: int, K: int, desc: lin_epi_desc | None,
                       num_cus: int) -> tuple[int, lin_epi_plan]:
    p = lin_epi_plan()
    d = ctypes.byref(desc) if desc is not None else None
    rc = load_library().lin_epi_query_plan(ctypes.c_void_p(handle or None), M, N, K, d, num_cus, ctypes.byref(p))
    return rc, p


def lin_epi_profile_read(handle: int) -> tuple[int, lin_epi_profile]:
    p = lin_epi_profile()
    rc = load_library().lin_epi_profile_read(ctypes.c_void_p(handle or None), ctypes.byref(p))
    return rc, p


def make_desc(kind: int, scale: float = 1.0, ht_min: float = -1.0, ht_max: float = 1.0, pool_kernel: int = 16,
              pool_stride: int | None = None) -> lin_epi_desc:
    return lin_epi_desc(int(kind), float(scale), float(ht_min), float(ht_max), int(pool_kernel),
                        int(pool_kernel if pool_stride is None else pool_stride))


def _check(rc: int, where: str) -> None:
    if rc != LIN_EPI_OK:
        raise LinEpiError(rc, where)


def _check_tensors(**tensors) -> None:
    import torch

    for name, t in tensors.items():
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float32 device tensor" % name)


class LinEpi:
    """A handle bound to a torch CUDA (HIP) stream; runs on torch tensors.

    ``run(X, W, b, desc)`` allocates Y with torch (device memory only) and
    calls lin_epi_run; the result is enqueued on the handle's stream.  Tensors
    the handle allocates come from torch's caching allocator on that stream,
    and input tensors are marked as used on it (``record_stream``) when the
    caller's current stream is another one, so the allocator does not hand
    their memory to other work before the handle's stream has finished with
    it.  A caller reading Y on another stream synchronises with the handle's
    stream first.
    """

    def __init__(self, stream=None):
        self.stream = stream
        ptr = stream.cuda_stream if stream is not None else 0
        rc, self.handle = lin_epi_create(ptr)
        _check(rc, "lin_epi_create")

    def _torch_stream(self, device):
        import torch

        return self.stream if self.stream is not None else torch.cuda.default_stream(device)

    def _alloc(self, shape, device):
        """An uninitialised float32 tensor owned by the handle's stream."""
        import torch

        with torch.cuda.stream(self._torch_stream(device)):
            return torch.empty(shape, dtype=torch.float32, device=device)

    def _mark_used(self, *tensors) -> None:
        import torch

        s = self._torch_stream(tensors[0].device)
        if torch.cuda.current_stream(tensors[0].device) != s:
            for t in tensors:
                t.record_stream(s)

    def close(self) -> None:
        if self.handle:
            rc = lin_epi_destroy(self.handle)
            self.handle = 0
            _check(rc, "lin_epi_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if self.handle:
                lin_epi_destroy(self.handle)
                self.handle = 0
        except Exception:
            pass

    def set_option(self, option: int, value: int) -> None:
        _check(lin_epi_set_option(self.handle, option, value), "lin_epi_set_option")

    def plan(self) -> lin_epi_plan:
        rc, p = lin_epi_last_plan(self.handle)
        _check(rc, "lin_epi_last_plan")
        return p

    def profile(self) -> lin_epi_profile:
        rc, p = lin_epi_profile_read(self.handle)
        _check(rc, "lin_epi_profile_read")
        return p

    @staticmethod
    def output_shape(M: int, N: int, kind: int) -> tuple:
        return (M,) if kind in (LIN_EPI_POOL_GELU_SCALE_ROWMAX, LIN_EPI_GELU_SCALE_ROWMAX) else (M, N)

    def scale_weights(self, W, b, scale: float):
        """Tail (a)'s scale folded into new weight and bias tensors."""
        _check_tensors(W=W, b=b)
        N, K = W.shape
        if tuple(b.shape) != (N,):
            raise ValueError("shape mismatch: W %s, b %s" % (tuple(W.shape), tuple(b.shape)))
        Ws = self._alloc((N, K), W.device)
        bs = self._alloc((N,), W.device)
        rc = lin_epi_scale_weights(self.handle, N, K, W.data_ptr(), b.data_ptr(), scale, Ws.data_ptr(), bs.data_ptr())
        _check(rc, "lin_epi_scale_weights")
        self._mark_used(W, b)
        return Ws, bs

    def pool_weights(self, W, b, pool_kernel: int = 16):
        """Window-averaged weights and bias (device tensors) for tail (b)."""
        _check_tensors(W=W, b=b)
        N, K = W.shape
        if tuple(b.shape) != (N,):
            raise ValueError("shape mismatch: W %s, b %s" % (tuple(W.shape), tuple(b.shape)))
        if pool_kernel <= 0:
            raise ValueError("pool_kernel must be positive")
        L = N // pool_kernel
        Wp = self._alloc((L, K), W.device)
        bp = self._alloc((L,), W.device)
        rc = lin_epi_pool_weights(self.handle, N, K, W.data_ptr(), b.data_ptr(), pool_kernel, Wp.data_ptr(),
                                  bp.data_ptr())
        _check(rc, "lin_epi_pool_weights")
        self._mark_used(W, b)
        return Wp, bp

    def run_into(self, X, W, b, desc: lin_epi_desc, Y) -> None:
        """lin_epi_run into a caller-allocated Y.  The fast path for repeated
        calls: beyond what the C ABI validates (sizes, alignment, kind) the
        caller guarantees contiguous float32 device tensors X [M,K], W [N,K],
        b [N] and Y of ``output_shape(M, N, kind)``; :meth:`run` checks them."""
        M, K = X.shape
        N = W.shape[0]
        rc = lin_epi_run(self.handle, M, N, K, X.data_ptr(), W.data_ptr(), b.data_ptr(), desc, Y.data_ptr())
        _check(rc, "lin_epi_run")

    def run(self, X, W, b, desc: lin_epi_desc):
        _check_tensors(X=X, W=W, b=b)
        M, K = X.shape
        N, K2 = W.shape
        if K2 != K or tuple(b.shape) != (N,):
            raise ValueError("shape mismatch: X %s, W %s, b %s" % (tuple(X.shape), tuple(W.shape), tuple(b.shape)))
        Y = self._alloc(self.output_shape(M, N, desc.kind), X.device)
        self.run_into(X, W, b, desc, Y)
        self._mark_used(X, W, b)
        return Y
