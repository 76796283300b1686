"""Python binding of libar (C ABI declared in include/ar.h).

Argument marshalling only: every step of the collective runs in libar's HIP
kernels.  The low-level functions carry the C names (``ar_init``,
``ar_allreduce``, ...) and take plain integers (device pointers, sizes,
stream handles).  ``Comm`` is a convenience wrapper over torch tensors:
PyTorch provides device memory and streams, nothing else.

There is no fallback: if ``libar.so`` has not been built, ``lib()`` raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libar.so")

# ---- constants mirrored from include/ar.h --------------------------------
AR_INT32, AR_FLOAT32, AR_BF16 = 0, 1, 2
AR_RING, AR_TREE, AR_AUTO = 0, 1, 2
AR_SIMPLE, AR_LL, AR_PROTO_AUTO = 0, 1, 2
AR_SUCCESS, AR_ERR_INVALID_ARG, AR_ERR_INVALID_USAGE, AR_ERR_UNSUPPORTED = 0, 1, 2, 3
AR_ERR_HIP, AR_ERR_TIMEOUT, AR_ERR_INTERNAL = 4, 5, 6
AR_LAUNCH_AUTO, AR_LAUNCH_STEP, AR_LAUNCH_FUSED, AR_LAUNCH_PIPELINED = 0, 1, 2, 3
(AR_OPT_CHUNK_BYTES, AR_OPT_LAUNCH, AR_OPT_GRID, AR_OPT_TIMEOUT_US, AR_OPT_DEBUG,
 AR_OPT_ALGO, AR_OPT_PROTO, AR_OPT_TREE_MAX_BYTES, AR_OPT_DEBUG_MUTE_RANK, AR_OPT_REDOP,
 AR_OPT_CHANNELS, AR_OPT_DEBUG_LL_LAUNCHES) = range(12)
AR_SUM, AR_MAX, AR_MIN, AR_AVG = 0, 1, 2, 3
(AR_COST_TREE_LL, AR_COST_RING_FUSED, AR_COST_RING_PIPELINED, AR_COST_RING_STEP,
 AR_COST_RING_LL, AR_COST_TREE_FUSED) = range(6)
COST_FORMS = {"tree-ll": AR_COST_TREE_LL, "ring-fused": AR_COST_RING_FUSED,
              "ring-pipelined": AR_COST_RING_PIPELINED, "ring-step": AR_COST_RING_STEP,
              "ring-ll": AR_COST_RING_LL, "tree-fused": AR_COST_TREE_FUSED}
REDOPS = {"sum": AR_SUM, "max": AR_MAX, "min": AR_MIN, "avg": AR_AVG}

DTYPES = {"int32": AR_INT32, "float32": AR_FLOAT32, "bf16": AR_BF16}
ALGOS = {"ring": AR_RING, "tree": AR_TREE, "auto": AR_AUTO}
PROTOS = {"simple": AR_SIMPLE, "ll": AR_LL, "auto": AR_PROTO_AUTO}
LAUNCHES = {"auto": AR_LAUNCH_AUTO, "step": AR_LAUNCH_STEP, "fused": AR_LAUNCH_FUSED,
            "pipelined": AR_LAUNCH_PIPELINED}
ELEM_SIZE = {AR_INT32: 4, AR_FLOAT32: 4, AR_BF16: 2}

_lib = None


class ArError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, ar_status_string(status), status))


def lib():
    """Load libar.so; raise if it is not built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libar.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    sig = {
        "ar_init": ([ctypes.POINTER(vp), i, sz, i, i, i], i),
        "ar_destroy": ([vp], i),
        "ar_workspace_bytes": ([vp], sz),
        "ar_set_workspace": ([vp, vp, sz, vp], i),
        "ar_allreduce": ([vp, vp, vp, sz, vp], i),
        "ar_allreduce_noalloc": ([vp, vp, vp, sz, vp], i),
        "ar_reduce_scatter": ([vp, vp, vp, sz, vp], i),
        "ar_all_gather": ([vp, vp, vp, sz, vp], i),
        "ar_check": ([vp], i),
        "ar_set_option": ([vp, i, i64], i),
        "ar_get_option": ([vp, i, ctypes.POINTER(i64)], i),
        "ar_plan": ([vp, sz, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)], i),
        "ar_set_cost": ([vp, i, ctypes.c_double, ctypes.c_double], i),
        "ar_get_cost": ([vp, i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], i),
        "ar_auto_tree_max_bytes": ([vp], i64),
        "ar_ring_segment": ([vp, sz, i, ctypes.POINTER(sz), ctypes.POINTER(sz)], i),
        "ar_tree_parent": ([vp, i, i], i),
        "ar_ring_channel_stride": ([vp, i], i),
        "ar_status_string": ([i], ctypes.c_char_p),
        "ar_last_hip_error": ([vp], i),
        "ar_stream_add": ([vp, vp, vp, sz, vp], i),
        "ar_stream_copy": ([vp, vp, sz, vp], i),
        "ar_stream_rows": ([vp, vp, i, sz, vp], i),
        "ar_ll_pingpong": ([vp, vp, i, i, i64, vp], i),
        "ar_stream_create_cu_masked": ([ctypes.POINTER(vp), ctypes.c_uint32,
                                        ctypes.POINTER(ctypes.c_uint32)], i),
        "ar_stream_destroy": ([vp], i),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _ok(status, what):
    if status != AR_SUCCESS:
        raise ArError(status, what)


# ---- the C entry points, same names ----------------------------------------

def ar_init(R, count, dtype, algo=AR_RING, proto=AR_SIMPLE):
    h = ctypes.c_void_p()
    _ok(lib().ar_init(ctypes.byref(h), R, count, dtype, algo, proto), "ar_init")
    return h.value


def ar_destroy(comm):
    return lib().ar_destroy(comm)


def ar_workspace_bytes(comm):
    return lib().ar_workspace_bytes(comm)


def ar_set_workspace(comm, dev_ptr, nbytes, stream=0):
    _ok(lib().ar_set_workspace(comm, dev_ptr, nbytes, stream), "ar_set_workspace")


def ar_allreduce(comm, send_ptr, recv_ptr, count, stream=0):
    _ok(lib().ar_allreduce(comm, send_ptr, recv_ptr, count, stream), "ar_allreduce")


def ar_allreduce_noalloc(comm, send_ptr, recv_ptr, count, stream=0):
    _ok(lib().ar_allreduce_noalloc(comm, send_ptr, recv_ptr, count, stream),
        "ar_allreduce_noalloc")


def ar_reduce_scatter(comm, send_ptr, recv_ptr, recvcount, stream=0):
    _ok(lib().ar_reduce_scatter(comm, send_ptr, recv_ptr, recvcount, stream), "ar_reduce_scatter")


def ar_all_gather(comm, send_ptr, recv_ptr, sendcount, stream=0):
    _ok(lib().ar_all_gather(comm, send_ptr, recv_ptr, sendcount, stream), "ar_all_gather")


def ar_check(comm):
    """Returns the status code (AR_SUCCESS or AR_ERR_TIMEOUT ...)."""
    return lib().ar_check(comm)


def ar_set_option(comm, option, value):
    _ok(lib().ar_set_option(comm, option, int(value)), "ar_set_option")


def ar_get_option(comm, option):
    v = ctypes.c_int64()
    _ok(lib().ar_get_option(comm, option, ctypes.byref(v)), "ar_get_option")
    return v.value


def ar_plan(comm, count):
    a, p, l = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _ok(lib().ar_plan(comm, count, ctypes.byref(a), ctypes.byref(p), ctypes.byref(l)), "ar_plan")
    return a.value, p.value, l.value


def ar_set_cost(comm, form, alpha_us, bw_gbps):
    _ok(lib().ar_set_cost(comm, form, alpha_us, bw_gbps), "ar_set_cost")


def ar_get_cost(comm, form):
    a, b = ctypes.c_double(), ctypes.c_double()
    _ok(lib().ar_get_cost(comm, form, ctypes.byref(a), ctypes.byref(b)), "ar_get_cost")
    return a.value, b.value


def ar_auto_tree_max_bytes(comm):
    return int(lib().ar_auto_tree_max_bytes(comm))


def ar_ring_segment(comm, count, c):
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    _ok(lib().ar_ring_segment(comm, count, c, ctypes.byref(lo), ctypes.byref(hi)),
        "ar_ring_segment")
    return lo.value, hi.value


def ar_tree_parent(comm, tree, r):
    return lib().ar_tree_parent(comm, tree, r)


def ar_ring_channel_stride(comm, k):
    return lib().ar_ring_channel_stride(comm, k)


def ar_status_string(status):
    return lib().ar_status_string(status).decode()


def ar_last_hip_error(comm):
    return lib().ar_last_hip_error(comm)


def ar_stream_add(a_ptr, b_ptr, c_ptr, n, stream=0):
    _ok(lib().ar_stream_add(a_ptr, b_ptr, c_ptr, n, stream), "ar_stream_add")


def ar_stream_copy(src_ptr, dst_ptr, nbytes, stream=0):
    _ok(lib().ar_stream_copy(src_ptr, dst_ptr, nbytes, stream), "ar_stream_copy")


def ar_stream_rows(src_ptr, dst_ptr, rows, row_bytes, stream=0):
    _ok(lib().ar_stream_rows(src_ptr, dst_ptr, rows, row_bytes, stream), "ar_stream_rows")


def ar_ll_pingpong(lines_ptr, result_ptr, iters, xcd_apart, timeout_us=2_000_000, stream=0):
    _ok(lib().ar_ll_pingpong(lines_ptr, result_ptr, iters, int(bool(xcd_apart)), timeout_us, stream),
        "ar_ll_pingpong")


def ar_stream_create_cu_masked(cus, num_cus):
    """A stream restricted to the CUs in `cus` (an iterable of CU indices);
    returns the raw hipStream_t as an integer."""
    words = (num_cus + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    rc = lib().ar_stream_create_cu_masked(ctypes.byref(h), words, mask)
    if rc != AR_SUCCESS:
        raise ArError(rc, "ar_stream_create_cu_masked (hipError %d)" % ar_last_hip_error(None))
    return h.value


def ar_stream_destroy(stream):
    _ok(lib().ar_stream_destroy(stream), "ar_stream_destroy")


# ---- torch convenience wrapper ---------------------------------------------

def _torch_dtype(dt):
    import torch
    return {AR_INT32: torch.int32, AR_FLOAT32: torch.float32, AR_BF16: torch.bfloat16}[dt]


class Comm:
    """A communicator of R logical ranks on one GPU, with its workspace.

    Buffers are rank-major torch tensors on the device: ``send`` of shape
    [R, n] etc.  Calls are asynchronous on the current torch stream (or the
    given one)."""

    def __init__(self, R, count, dtype="float32", algo="ring", proto="simple", device=None,
                 launch=None, **options):
        import torch
        self.R = R
        self.count = count
        self.dtype = DTYPES[dtype] if isinstance(dtype, str) else dtype
        self.device = torch.device(device if device is not None else "cuda")
        self.handle = ar_init(R, count, self.dtype,
                              ALGOS[algo] if isinstance(algo, str) else algo,
                              PROTOS[proto] if isinstance(proto, str) else proto)
        if launch is not None:
            self.set_option(AR_OPT_LAUNCH, LAUNCHES[launch] if isinstance(launch, str) else launch)
        for k, v in options.items():
            if k == "redop" and isinstance(v, str):
                v = REDOPS[v]
            self.set_option(globals()["AR_OPT_" + k.upper()], v)
        nbytes = ar_workspace_bytes(self.handle)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self._ws_stream = torch.cuda.current_stream(self.device).cuda_stream
        ar_set_workspace(self.handle, self.workspace.data_ptr(), self.workspace.numel(),
                         self._stream(None))

    def _stream(self, stream):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if getattr(self, "workspace", None) is not None and \
                s.cuda_stream != self._ws_stream and not torch.cuda.is_current_stream_capturing():
            # the workspace may still be in use on this stream when the comm is
            # dropped: keep torch's allocator from reusing it too early
            self.workspace.record_stream(s)
        return s.cuda_stream

    def _check_tensor(self, t, rows, cols, what):
        if t.device != self.device and not (t.is_cuda and self.device.index is None):
            raise ValueError("%s must be on %s" % (what, self.device))
        if t.dtype != _torch_dtype(self.dtype):
            raise ValueError("%s has dtype %s, comm has %s" % (what, t.dtype, _torch_dtype(self.dtype)))
        if tuple(t.shape) != (rows, cols):
            raise ValueError("%s must have shape (%d, %d), got %s" % (what, rows, cols, tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (rank-major rows)" % what)

    def allreduce(self, send, recv, stream=None):
        n = send.shape[1]
        self._check_tensor(send, self.R, n, "send")
        self._check_tensor(recv, self.R, n, "recv")
        ar_allreduce(self.handle, send.data_ptr(), recv.data_ptr(), n, self._stream(stream))
        return recv

    def reduce_scatter(self, send, recv, stream=None):
        n = recv.shape[1]
        self._check_tensor(send, self.R, n * self.R, "send")
        self._check_tensor(recv, self.R, n, "recv")
        ar_reduce_scatter(self.handle, send.data_ptr(), recv.data_ptr(), n, self._stream(stream))
        return recv

    def all_gather(self, send, recv, stream=None):
        n = send.shape[1]
        self._check_tensor(send, self.R, n, "send")
        self._check_tensor(recv, self.R, n * self.R, "recv")
        ar_all_gather(self.handle, send.data_ptr(), recv.data_ptr(), n, self._stream(stream))
        return recv

    def check(self):
        return ar_check(self.handle)

    def set_option(self, option, value):
        ar_set_option(self.handle, option, value)

    def get_option(self, option):
        return ar_get_option(self.handle, option)

    def plan(self, count):
        return ar_plan(self.handle, count)

    def channel_strides(self):
        """Ring stride of each channel this comm runs."""
        K = self.get_option(AR_OPT_CHANNELS)
        return [ar_ring_channel_stride(self.handle, k) for k in range(K)]

    def close(self):
        """Destroy the communicator and release its workspace.  A comm used on
        a stream that the caller destroys itself (ar_stream_destroy) must be
        closed, and that stream's work finished, before the stream goes: the
        workspace is recorded on every stream the comm ran on."""
        if getattr(self, "handle", None):
            ar_destroy(self.handle)
            self.handle = None
        self.workspace = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
