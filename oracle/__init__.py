"""CPU oracle for ring / double-binary-tree all-reduce, reduce-scatter and
all-gather over R logical ranks -- a thin ctypes wrapper over ``oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports it, and it imports nothing from the GPU library.

Arrays are numpy, rank-major ``[R, N]``.  bfloat16 arrays are carried as
``uint16`` bit patterns and named by ``dtype="bf16"``.
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_DT = {"int32": 0, "float32": 1, "bf16": 2}
OPS = {"sum": 0, "max": 1, "min": 2, "avg": 3}
_NP = {"int32": np.int32, "float32": np.float32, "bf16": np.uint16}
_libs = {}
_use_omp = False


@contextlib.contextmanager
def parallel(threads):
    """Inside the block, oracle calls run on the OpenMP build of the same
    code with `threads` threads (parallel over elements within each step;
    every element keeps its summation order, so the results are the same
    bits).  Yields the number of threads OpenMP reports it will use."""
    global _use_omp
    prev = _use_omp
    _use_omp = True
    try:
        yield int(lib().orc_set_threads(int(threads)))
    finally:
        _use_omp = prev


def lib():
    """Load the oracle library (the OpenMP build inside `parallel()`, else the
    single-threaded one), compiling both first only if either is missing."""
    path = _build.LIB_OMP if _use_omp else _build.LIB
    if path not in _libs:
        if not (os.path.exists(_build.LIB) and os.path.exists(_build.LIB_OMP)):
            _build.build()
        L = ctypes.CDLL(path)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        for name in ("orc_ring_allreduce", "orc_ring_reduce_scatter",
                     "orc_ring_all_gather", "orc_tree_allreduce"):
            f = getattr(L, name)
            f.argtypes = [i, sz, i, vp, vp]
            f.restype = i
        for name in ("orc_ring_allreduce_op", "orc_ring_reduce_scatter_op",
                     "orc_tree_allreduce_op"):
            f = getattr(L, name)
            f.argtypes = [i, sz, i, i, vp, vp]
            f.restype = i
        for name in ("orc_ring_allreduce_ch", "orc_ring_reduce_scatter_ch"):
            f = getattr(L, name)
            f.argtypes = [i, sz, i, i, i, vp, vp, vp]
            f.restype = i
        L.orc_ring_all_gather_ch.argtypes = [i, sz, i, i, vp, vp, vp]
        L.orc_ring_all_gather_ch.restype = i
        L.orc_exact_sum.argtypes = [i, sz, i, vp, vp]
        L.orc_exact_sum.restype = i
        L.orc_tree_parent.argtypes = [i, i, i]
        L.orc_tree_parent.restype = i
        L.orc_bf16_from_f32.argtypes = [ctypes.c_float]
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.orc_f32_from_bf16.restype = ctypes.c_float
        L.orc_bf16_from_f32_array.argtypes = [vp, vp, sz]
        L.orc_bf16_from_f32_array.restype = None
        L.orc_set_threads.argtypes = [i]
        L.orc_set_threads.restype = i
        _libs[path] = L
    return _libs[path]


def _dtype_of(x, dtype):
    if dtype is None:
        if x.dtype == np.int32:
            return "int32"
        if x.dtype == np.float32:
            return "float32"
        raise ValueError("pass dtype='bf16' for uint16 bfloat16 arrays")
    if dtype not in _DT:
        raise ValueError("unknown dtype %r" % (dtype,))
    return dtype


def _prep(x, dtype):
    dtype = _dtype_of(x, dtype)
    x = np.ascontiguousarray(x, dtype=_NP[dtype])
    if x.ndim != 2 or x.shape[0] < 2:
        raise ValueError("expected a rank-major [R, N] array with R >= 2")
    return x, dtype


def _check(rc, name):
    if rc != 0:
        raise RuntimeError("%s failed with code %d" % (name, rc))


def _strides(strides):
    strides = [1] if strides is None else list(strides)
    return len(strides), (ctypes.c_int * len(strides))(*strides)


def ring_allreduce(x, dtype=None, op="sum", strides=None):
    """Ring all-reduce: every row of the result is the reduction over ranks,
    folded in the ring's order (left fold from the owner's successor); for
    "avg" the owner divides the sum by R once.  `strides` lists one ring
    stride per channel (default: one channel, stride 1)."""
    x, dtype = _prep(x, dtype)
    R, N = x.shape
    y = np.empty_like(x)
    K, m = _strides(strides)
    _check(lib().orc_ring_allreduce_ch(R, N, _DT[dtype], OPS[op], K, m, x.ctypes.data,
                                       y.ctypes.data), "orc_ring_allreduce_ch")
    return y


def ring_reduce_scatter(x, dtype=None, op="sum", strides=None):
    """Ring reduce-scatter: rank q gets segment q of the reduction; [R, N/R]."""
    x, dtype = _prep(x, dtype)
    R, N = x.shape
    if N % R:
        raise ValueError("reduce-scatter needs N divisible by R")
    y = np.empty((R, N // R), dtype=x.dtype)
    K, m = _strides(strides)
    _check(lib().orc_ring_reduce_scatter_ch(R, N, _DT[dtype], OPS[op], K, m, x.ctypes.data,
                                            y.ctypes.data), "orc_ring_reduce_scatter_ch")
    return y


def ring_all_gather(shards, dtype=None, strides=None):
    """Ring all-gather: [R, n] shards -> [R, R*n], every row [x0, ..., x_{R-1}]."""
    x, dtype = _prep(shards, dtype)
    R, n = x.shape
    y = np.empty((R, R * n), dtype=x.dtype)
    K, m = _strides(strides)
    _check(lib().orc_ring_all_gather_ch(R, n, _DT[dtype], K, m, x.ctypes.data, y.ctypes.data),
           "orc_ring_all_gather_ch")
    return y


def tree_allreduce(x, dtype=None, op="sum"):
    """Double-binary-tree all-reduce: first half of the elements through tree
    A, second half through tree B; fold = own value, then children in
    ascending rank order; for "avg" the root divides the sum by R once."""
    x, dtype = _prep(x, dtype)
    R, N = x.shape
    y = np.empty_like(x)
    _check(lib().orc_tree_allreduce_op(R, N, _DT[dtype], OPS[op], x.ctypes.data, y.ctypes.data),
           "orc_tree_allreduce_op")
    return y


def exact_sum(x, dtype=None):
    """Plain definition: float64 sum over ranks, per element; shape [N]."""
    x, dtype = _prep(x, dtype)
    R, N = x.shape
    out = np.empty(N, dtype=np.float64)
    _check(lib().orc_exact_sum(R, N, _DT[dtype], x.ctypes.data, out.ctypes.data),
           "orc_exact_sum")
    return out


def tree_parents(R, tree):
    """Parent of every rank in tree 0 (A) or 1 (B); -1 marks the root."""
    return [lib().orc_tree_parent(R, tree, r) for r in range(R)]


def bf16_from_f32(a):
    """float32 array -> bfloat16 bit patterns (uint16), nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_bf16_from_f32_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_from_bf16(h):
    """bfloat16 bit patterns -> float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)

