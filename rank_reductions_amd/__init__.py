"""Python binding of librankred.so: collectives over R logical ranks on one GPU.

Argument marshalling only.  Every collective runs in the library's HIP
kernels; PyTorch supplies device memory and streams.  The functions mirror the
public tensor collective API of the ruCCL README (ja), user guide section 2
(register, all_reduce, reduce, broadcast, finish_collective, reset_collective),
plus reduce_scatter_tensor and all_gather_into_tensor of the monarch
Communicator page, a whole-gradient all_reduce_many and the parameter-keyed
gradient sync all_reduce_params (section 6, "Collective training"), and a
per-rank front end (rank_*) in which each logical rank calls from its own
thread.

    import rank_reductions_amd as rr
    rr.register(4)
    outs = rr.all_reduce(xs, op="sum")     # xs: 4 CUDA tensors, same shape
    rr.finish()

Errors from the library raise CollectiveError with the status code and text.
If librankred.so is not built the module still imports, but every call raises
(there is no fallback path).
"""

import ctypes
import threading
from pathlib import Path

import numpy as np

__all__ = [
    "CollectiveError", "register", "all_reduce", "reduce", "broadcast", "reduce_scatter",
    "all_gather", "all_reduce_many", "finish", "reset", "library", "library_path",
    "RC_OK", "RC_ERR_NOT_REGISTERED", "RC_ERR_DUPLICATE_REGISTRATION", "RC_ERR_SHAPE_MISMATCH",
    "RC_ERR_OP_MISMATCH", "RC_ERR_ROOT_MISMATCH", "RC_ERR_BROADCAST_SENDERS",
    "RC_ERR_DTYPE_MISMATCH", "RC_ERR_INVALID_ARGUMENT", "RC_ERR_DEVICE", "RC_ERR_PARAM_MISMATCH",
    "all_reduce_many_static", "all_reduce_params", "rank_register", "rank_finish", "rank_all_reduce", "rank_reduce",
    "rank_broadcast", "rank_reduce_scatter", "rank_all_gather", "rank_all_reduce_params",
    "all_gather_list", "all_to_all_single", "send_recv", "barrier", "rank_all_gather_list",
    "rank_all_to_all_single", "rank_send", "rank_recv", "rank_barrier", "rank_split", "rank_split_all",
    "Communicator",
]

RC_MAX_RANKS = 16
RC_ABI_VERSION = 3  # the include/rc.h this binding is written against
RC_MAX_DIMS = 8

RC_F32, RC_I32 = 0, 1
RC_SUM, RC_MEAN, RC_MAX = 0, 1, 2
RC_ALGO_AUTO, RC_ALGO_DIRECT, RC_ALGO_RING = 0, 1, 2
RC_CACHE_AUTO, RC_CACHE_STREAMING, RC_CACHE_NORMAL = 0, 1, 2

RC_OK = 0
RC_ERR_NOT_REGISTERED = 1
RC_ERR_DUPLICATE_REGISTRATION = 2
RC_ERR_SHAPE_MISMATCH = 3
RC_ERR_OP_MISMATCH = 4
RC_ERR_ROOT_MISMATCH = 5
RC_ERR_BROADCAST_SENDERS = 6
RC_ERR_DTYPE_MISMATCH = 7
RC_ERR_INVALID_ARGUMENT = 8
RC_ERR_DEVICE = 9
RC_ERR_PARAM_MISMATCH = 10

OPS = {"sum": RC_SUM, "mean": RC_MEAN, "max": RC_MAX}
ALGOS = {"auto": RC_ALGO_AUTO, "direct": RC_ALGO_DIRECT, "ring": RC_ALGO_RING}
CACHE_HINTS = {"auto": RC_CACHE_AUTO, "streaming": RC_CACHE_STREAMING, "normal": RC_CACHE_NORMAL}


class RcBuf(ctypes.Structure):
    _fields_ = [
        ("send", ctypes.c_void_p),
        ("recv", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("op", ctypes.c_int32),
        ("root", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("dims", ctypes.c_int64 * RC_MAX_DIMS),
    ]


class RcConfig(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("device", ctypes.c_int32),
        ("algo", ctypes.c_int32),
        ("validate_only", ctypes.c_int32),
        ("tile_elems", ctypes.c_int64),
        ("max_workgroups", ctypes.c_int32),
        ("cache_hint", ctypes.c_int32),
        ("waves_per_cu", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class RcParam(ctypes.Structure):
    """One rank's entry of a gradient sync: parameter ID, optional
    accumulator, and the gradient's rc_buf."""
    _fields_ = [("id", ctypes.c_uint64), ("acc", ctypes.c_void_p), ("buf", RcBuf)]


# numpy view of rc_buf, for building large batches quickly
RCBUF_NP = np.dtype([("send", "<u8"), ("recv", "<u8"), ("dtype", "<i4"), ("op", "<i4"),
                     ("root", "<i4"), ("ndim", "<i4"), ("dims", "<i8", (RC_MAX_DIMS,))])
assert RCBUF_NP.itemsize == ctypes.sizeof(RcBuf)


class CollectiveError(RuntimeError):
    """A status other than RC_OK from librankred (the CollectiveError cases of
    the ruCCL README, section 4, plus invalid-argument and device errors)."""

    def __init__(self, code, message):
        self.code = code
        self.name = _status_name(code)
        super().__init__(f"{self.name}: {message}")


def library_path():
    return Path(__file__).resolve().with_name("librankred.so")


_lib = None
_lib_lock = threading.Lock()


def library():
    """The loaded librankred.so (ctypes), loading it on first use.  Raises if
    it is not built or was built from another version of include/rc.h."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is None:
            _lib = _load()
    return _lib


def _load():
    path = library_path()
    if not path.exists():
        raise RuntimeError(f"{path} is not built: run `python -m rank_reductions_amd.build` "
                           "(no fallback implementation exists)")
    lib = ctypes.CDLL(str(path))
    lib.rc_abi_version.argtypes = []
    lib.rc_abi_version.restype = ctypes.c_int
    if lib.rc_abi_version() != RC_ABI_VERSION:
        raise RuntimeError(f"{path} reports ABI version {lib.rc_abi_version()}, this binding expects "
                           f"{RC_ABI_VERSION}: rebuild with `python -m rank_reductions_amd.build`")
    for name in ("rc_all_reduce", "rc_reduce", "rc_broadcast", "rc_reduce_scatter", "rc_all_gather"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.rc_register.argtypes = [ctypes.c_int, ctypes.POINTER(RcConfig)]
    lib.rc_register.restype = ctypes.c_int
    for name in ("rc_all_reduce_many", "rc_all_reduce_many_static"):
        getattr(lib, name).argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("rc_finish", "rc_reset", "rc_abi_version"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_int
    lib.rc_last_error.argtypes = []
    lib.rc_last_error.restype = ctypes.c_char_p
    lib.rc_status_name.argtypes = [ctypes.c_int]
    lib.rc_status_name.restype = ctypes.c_char_p
    lib.rc_rank_register.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(RcConfig)]
    lib.rc_rank_register.restype = ctypes.c_int
    for name in ("rc_rank_all_reduce", "rc_rank_reduce", "rc_rank_broadcast", "rc_rank_reduce_scatter",
                 "rc_rank_all_gather"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.rc_all_reduce_params.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_all_reduce_params.restype = ctypes.c_int
    lib.rc_rank_all_reduce_params.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_rank_all_reduce_params.restype = ctypes.c_int
    lib.rc_all_gather_list.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_all_gather_list.restype = ctypes.c_int
    lib.rc_all_to_all_single.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_all_to_all_single.restype = ctypes.c_int
    lib.rc_send_recv.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_send_recv.restype = ctypes.c_int
    lib.rc_barrier.argtypes = [ctypes.c_void_p]
    lib.rc_barrier.restype = ctypes.c_int
    lib.rc_rank_all_gather_list.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_rank_all_gather_list.restype = ctypes.c_int
    lib.rc_rank_all_to_all_single.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.rc_rank_all_to_all_single.restype = ctypes.c_int
    for name in ("rc_rank_send", "rc_rank_recv"):
        getattr(lib, name).argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    lib.rc_rank_barrier.argtypes = [ctypes.c_int, ctypes.c_void_p]
    lib.rc_rank_barrier.restype = ctypes.c_int
    lib.rc_rank_split.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    lib.rc_rank_split.restype = ctypes.c_int
    lib.rc_rank_finish.argtypes = [ctypes.c_int]
    lib.rc_rank_finish.restype = ctypes.c_int
    return lib


def _status_name(code):
    try:
        return library().rc_status_name(code).decode()
    except Exception:  # noqa: BLE001 - naming only
        return f"status {code}"


def check(code):
    """Raise CollectiveError for a non-RC_OK status."""
    if code != RC_OK:
        raise CollectiveError(code, library().rc_last_error().decode())
    return code


# ---------------------------------------------------------------- raw layer

def make_config(device=-1, algo="auto", validate_only=False, tile_elems=0, max_workgroups=0,
                cache_hint="auto", waves_per_cu=0):
    cfg = RcConfig()
    cfg.struct_size = ctypes.sizeof(RcConfig)
    cfg.device = device
    cfg.algo = ALGOS[algo] if isinstance(algo, str) else int(algo)
    cfg.validate_only = 1 if validate_only else 0
    cfg.tile_elems = tile_elems
    cfg.max_workgroups = max_workgroups
    cfg.cache_hint = CACHE_HINTS[cache_hint] if isinstance(cache_hint, str) else int(cache_hint)
    cfg.waves_per_cu = waves_per_cu
    return cfg


def make_bufs(sends, recvs, shape, dtype=RC_F32, op=RC_SUM, root=0):
    """An rc_buf array from raw addresses (ints or None); shape may be one
    tuple for all ranks or a list of per-rank tuples."""
    n = len(sends)
    arr = (RcBuf * n)()
    for r in range(n):
        shp = shape[r] if shape and isinstance(shape[0], (tuple, list)) else shape
        b = arr[r]
        b.send = sends[r] if sends[r] else None
        b.recv = recvs[r] if recvs[r] else None
        b.dtype = dtype[r] if isinstance(dtype, (list, tuple)) else dtype
        b.op = op[r] if isinstance(op, (list, tuple)) else op
        b.root = root[r] if isinstance(root, (list, tuple)) else root
        b.ndim = len(shp)
        for d, v in enumerate(shp):
            b.dims[d] = v
    return arr


def register(num_ranks, device=None, algo="auto", validate_only=False, tile_elems=0,
             max_workgroups=0, cache_hint="auto", waves_per_cu=0):
    """register<B>: open the process-wide session for num_ranks logical ranks."""
    if device is None:
        device = -1
    elif not isinstance(device, int):
        import torch
        device = torch.device(device).index if torch.device(device).index is not None else -1
    cfg = make_config(device, algo, validate_only, tile_elems, max_workgroups, cache_hint, waves_per_cu)
    return check(library().rc_register(int(num_ranks), ctypes.byref(cfg)))


def finish():
    """finish_collective<B>: wait for the GPU, free scratch, close the session."""
    return check(library().rc_finish())


def reset():
    """reset_collective<B>: drop the registration and in-flight state."""
    return check(library().rc_reset())


# ---------------------------------------------------------------- torch layer

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return RC_F32
    if t.dtype == torch.int32:
        return RC_I32
    raise TypeError(f"unsupported dtype {t.dtype}; float32 and int32 are supported")


# Address passed for a zero-element tensor whose storage pointer is NULL: the
# library never dereferences it (count 0), but a broadcast sender must be
# non-NULL to be recognised.
_EMPTY_ADDR = 256


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on a CUDA (HIP) device")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    p = t.data_ptr()
    return p if p or t.numel() else _EMPTY_ADDR


def _expect(out, ref, numel, what):
    """Checks an output tensor the library writes `numel` elements of ref's
    dtype into: the C ABI carries the input's shape only, so an undersized or
    mistyped output would be written past its end or misread.  Raises
    CollectiveError before anything is launched."""
    if out is None:
        raise CollectiveError(RC_ERR_INVALID_ARGUMENT, f"{what}: no output tensor")
    if out.dtype != ref.dtype:
        raise CollectiveError(RC_ERR_DTYPE_MISMATCH, f"{what}: output dtype {out.dtype}, input dtype {ref.dtype}")
    if out.numel() != numel:
        raise CollectiveError(RC_ERR_SHAPE_MISMATCH,
                              f"{what}: output holds {out.numel()} elements, the call writes {numel}")
    if out.device != ref.device:
        raise CollectiveError(RC_ERR_INVALID_ARGUMENT, f"{what}: output on {out.device}, input on {ref.device}")
    if not out.is_contiguous():
        raise CollectiveError(RC_ERR_INVALID_ARGUMENT, f"{what}: output is not contiguous")


def _expect_list(outs, n, what):
    if len(outs) != n:
        raise CollectiveError(RC_ERR_INVALID_ARGUMENT, f"{what}: {len(outs)} outputs for {n} ranks")


def _stream(stream, ref):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    torch = _torch()
    return torch.cuda.current_stream(ref.device).cuda_stream


def _op(op):
    return OPS[op] if isinstance(op, str) else int(op)


def _call(fn, sends, recvs, op=RC_SUM, root=0, stream=None, shapes=None):
    """One rc_* call: per-rank dtype and shape come from each rank's send
    tensor (or its recv tensor where send is None), so the library sees and
    checks every rank's own description."""
    descr = [s if s is not None else r for s, r in zip(sends, recvs)]
    ref = next((t for t in descr if t is not None), None)
    if ref is None:
        raise ValueError("no tensor given")
    if shapes is None:
        shapes = [tuple(t.shape) if t is not None else () for t in descr]
    dtypes = [_dtype_code(t) if t is not None else RC_F32 for t in descr]
    bufs = make_bufs([_ptr(s) for s in sends], [_ptr(r) for r in recvs], shapes, dtypes, op, root)
    check(fn(ctypes.cast(bufs, ctypes.c_void_p), ctypes.c_void_p(_stream(stream, ref))))


def all_reduce(xs, op="sum", out=None, stream=None):
    """all_reduce<B>: every rank receives the reduction of all ranks' tensors.
    Returns the R output tensors (new ones unless `out` is given; out may be
    `xs` itself for in place)."""
    torch = _torch()
    if out is None:
        out = [torch.empty_like(x) for x in xs]
    _expect_list(out, len(xs), "all_reduce")
    for r, (x, o) in enumerate(zip(xs, out)):
        _expect(o, x, x.numel(), f"all_reduce rank {r}")
    _call(library().rc_all_reduce, xs, out, _op(op), 0, stream)
    return out


def reduce(xs, root, op="sum", out=None, stream=None):
    """reduce<B>: only `root` receives the reduction; other entries are None."""
    torch = _torch()
    if out is None:
        out = [torch.empty_like(xs[root]) if r == root else None for r in range(len(xs))]
    _expect_list(out, len(xs), "reduce")
    if 0 <= root < len(xs):  # a root out of range is the library's to report
        _expect(out[root], xs[root], xs[root].numel(), f"reduce root {root}")
    _call(library().rc_reduce, xs, out, _op(op), root, stream)
    return out


def broadcast(sends, out=None, stream=None, root=-1):
    """broadcast<B>: exactly one entry of `sends` is a tensor (the sender),
    the others are None; every rank receives the sender's bytes."""
    torch = _torch()
    senders = [s for s in sends if s is not None]
    ref = senders[0] if senders else None
    if ref is None:
        raise CollectiveError(RC_ERR_BROADCAST_SENDERS, "broadcast needs one sender tensor")
    if out is None:
        out = [torch.empty_like(ref) if s is None else None for s in sends]
    _expect_list(out, len(sends), "broadcast")
    for r, (snd, o) in enumerate(zip(sends, out)):
        if o is not None and (snd is None or o is not snd):
            _expect(o, ref, ref.numel(), f"broadcast rank {r}")
    _call(library().rc_broadcast, sends, out, RC_SUM, root, stream)
    return out


def reduce_scatter(xs, op="sum", out=None, stream=None):
    """reduce_scatter_tensor: rank r receives shard r (count/R elements) of the
    reduction of the ranks' flat inputs."""
    torch = _torch()
    R = len(xs)
    if out is None:
        out = [torch.empty(x.numel() // R, dtype=x.dtype, device=x.device) for x in xs]
    _expect_list(out, R, "reduce_scatter")
    for r, (x, o) in enumerate(zip(xs, out)):
        if x.numel() % R == 0:  # an indivisible count is the library's to report
            _expect(o, x, x.numel() // R, f"reduce_scatter rank {r}")
    _call(library().rc_reduce_scatter, xs, out, _op(op), 0, stream)
    return out


def all_gather(shards, out=None, stream=None):
    """all_gather_into_tensor: every rank receives the R shards concatenated
    in rank order."""
    torch = _torch()
    R = len(shards)
    if out is None:
        out = [torch.empty(R * s.numel(), dtype=s.dtype, device=s.device) for s in shards]
    _expect_list(out, R, "all_gather")
    for r, (x, o) in enumerate(zip(shards, out)):
        _expect(o, x, R * x.numel(), f"all_gather rank {r}")
    _call(library().rc_all_gather, shards, out, RC_SUM, 0, stream)
    return out


def batch_bufs(tensors, outs, op):
    """rc_buf rows [num_tensors][num_ranks] as a numpy structured array; every
    output is checked against its input first."""
    T = len(tensors)
    R = len(tensors[0]) if T else 0
    _expect_list(outs, T, "batched all_reduce (tensors)")
    for t in range(T):
        _expect_list(outs[t], len(tensors[t]), f"batched all_reduce tensor {t}")
        for r in range(len(tensors[t])):
            _expect(outs[t][r], tensors[t][r], tensors[t][r].numel(), f"batched all_reduce tensor {t} rank {r}")
    arr = np.zeros(T * R, dtype=RCBUF_NP)
    k = 0
    for t in range(T):
        for r in range(R):
            x = tensors[t][r]
            y = outs[t][r]
            arr[k]["send"] = _ptr(x)
            arr[k]["recv"] = _ptr(y)
            arr[k]["dtype"] = _dtype_code(x)
            arr[k]["op"] = op
            arr[k]["ndim"] = x.dim()
            arr[k]["dims"][:x.dim()] = x.shape
            k += 1
    return arr


def all_reduce_many(tensors, op="mean", out=None, stream=None):
    """Whole-gradient all-reduce: tensors[t][r] is rank r's copy of tensor t.
    Each tensor is reduced as rc_all_reduce would, in few launches.
    Returns out[t][r]."""
    torch = _torch()
    if out is None:
        out = [[torch.empty_like(x) for x in per_rank] for per_rank in tensors]
    if not tensors:
        return out
    arr = batch_bufs(tensors, out, _op(op))
    ref = tensors[0][0]
    check(library().rc_all_reduce_many(len(tensors), ctypes.c_void_p(arr.ctypes.data),
                                       ctypes.c_void_p(_stream(stream, ref))))
    return out


def all_reduce_many_static(tensors, op="mean", out=None, stream=None):
    """all_reduce_many for callers that cannot allocate device memory (graph
    capture, serving loops): the batched tensors' descriptor tables go to the
    library's static device scratch (1 MiB per GPU) instead of its arena, and
    only kernels are enqueued.  Same bits as all_reduce_many.  Calls that
    overlap on one GPU race on the scratch."""
    torch = _torch()
    if out is None:
        out = [[torch.empty_like(x) for x in per_rank] for per_rank in tensors]
    if not tensors:
        return out
    arr = batch_bufs(tensors, out, _op(op))
    ref = tensors[0][0]
    check(library().rc_all_reduce_many_static(len(tensors), ctypes.c_void_p(arr.ctypes.data),
                                              ctypes.c_void_p(_stream(stream, ref))))
    return out


def all_gather_list(shards, out=None, stream=None):
    """Communicator.all_gather, the list form: out[r][k] receives rank k's
    shard on every rank r (allocated when out is None)."""
    torch = _torch()
    R = len(shards)
    if out is None:
        out = [[torch.empty_like(shards[k]) for k in range(R)] for _ in range(R)]
    _expect_list(out, R, "all_gather_list")
    for r in range(R):
        _expect_list(out[r], R, f"all_gather_list rank {r}")
        for k in range(R):
            _expect(out[r][k], shards[k], shards[k].numel(), f"all_gather_list rank {r} shard {k}")
    bufs = make_bufs([_ptr(x) for x in shards], [None] * R, [tuple(x.shape) for x in shards],
                     [_dtype_code(x) for x in shards])
    recvs = (ctypes.c_void_p * (R * R))(*[_ptr(out[r][k]) for r in range(R) for k in range(R)])
    check(library().rc_all_gather_list(ctypes.cast(bufs, ctypes.c_void_p), recvs,
                                       ctypes.c_void_p(_stream(stream, shards[0]))))
    return out


def all_to_all_single(xs, out=None, stream=None):
    """Communicator.all_to_all_single: rank d's output holds, in source-rank
    order, split d of every rank's input (equal splits of N/R elements)."""
    torch = _torch()
    if out is None:
        out = [torch.empty_like(x) for x in xs]
    _expect_list(out, len(xs), "all_to_all_single")
    for r, (x, o) in enumerate(zip(xs, out)):
        _expect(o, x, x.numel(), f"all_to_all_single rank {r}")
    _call(library().rc_all_to_all_single, xs, out, stream=stream)
    return out


def send_recv(x, src, dst, out=None, stream=None):
    """Communicator.send on rank src and recv on rank dst, as one call: out
    (rank dst's tensor) receives x (rank src's)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    _expect(out, x, x.numel(), "send_recv")
    bufs = make_bufs([_ptr(x), None], [None, _ptr(out)], [tuple(x.shape), tuple(out.shape)],
                     [_dtype_code(x), _dtype_code(out)])
    check(library().rc_send_recv(int(src), int(dst), ctypes.cast(bufs, ctypes.c_void_p),
                                 ctypes.c_void_p(_stream(stream, x))))
    return out


def barrier(stream=None):
    """Communicator.barrier for the whole-call form (one stream: nothing to join)."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else (int(stream) if stream else 0)
    return check(library().rc_barrier(ctypes.c_void_p(s)))


def _param_entries(grads, outs, op, acc=None):
    """One rank's map as an rc_param array (in the map's order) and its length;
    outputs and accumulators are checked against their gradients first."""
    keys = list(grads)
    n = len(keys)
    for k in keys:
        if k not in outs:
            raise CollectiveError(RC_ERR_INVALID_ARGUMENT, f"all_reduce_params: no output for parameter {k}")
        _expect(outs[k], grads[k], grads[k].numel(), f"all_reduce_params output of parameter {k}")
        a = acc.get(k) if acc else None
        if a is not None:
            _expect(a, grads[k], grads[k].numel(), f"all_reduce_params accumulator of parameter {k}")
    arr = (RcParam * max(n, 1))()
    if n:
        bufs = make_bufs([_ptr(grads[k]) for k in keys], [_ptr(outs[k]) for k in keys],
                         [tuple(grads[k].shape) for k in keys], [_dtype_code(grads[k]) for k in keys], op)
        for i, k in enumerate(keys):
            arr[i].id = int(k)
            a = acc.get(k) if acc else None
            arr[i].acc = _ptr(a) if a is not None else None
            arr[i].buf = bufs[i]
    return n, arr


def _first_tensor(maps):
    return next((v for m in maps for v in m.values()), None)


def _stream_for(stream, ref):
    if ref is not None:
        return _stream(stream, ref)
    return _stream(stream, None) if stream is not None else 0


def all_reduce_params(grads, op="mean", out=None, stream=None, acc=None):
    """Gradient sync keyed by parameter ID (ruCCL README section 6,
    grads.all_reduce_with(communicator, ReduceOperation::Mean)).  grads[r] is
    rank r's map {parameter id: CUDA tensor}; entries pair across ranks by ID,
    whatever order each map lists them in.  acc, if given, is one map per rank
    of accumulated gradients (a GradientsAccumulator's sum over earlier
    microbatches): a parameter with one is reduced over acc + grad, fused into
    the same pass.  Returns out: one map per rank with the reduced tensors
    (allocated when out is None; out may be grads or acc, in place).
    Different ID sets raise CollectiveError with RC_ERR_PARAM_MISMATCH."""
    torch = _torch()
    R = len(grads)
    if out is None:
        out = [{k: torch.empty_like(v) for k, v in g.items()} for g in grads]
    accs = acc if acc is not None else [None] * R
    entries = [_param_entries(g, o, _op(op), a) for g, o, a in zip(grads, out, accs)]
    counts = (ctypes.c_int * R)(*[e[0] for e in entries])
    params = (ctypes.c_void_p * R)(*[ctypes.addressof(e[1]) for e in entries])
    s = _stream_for(stream, _first_tensor(grads))
    check(library().rc_all_reduce_params(counts, params, ctypes.c_void_p(s)))
    return out


# ---------------------------------------------------------------- per-rank front end
#
# Each logical rank calls these from its own thread with its own tensors and
# stream; the k-th calls of all ranks form one collective (ruCCL README,
# section 3).  Every call blocks until all ranks have made theirs.

def rank_register(rank, num_ranks, device=None, **cfg):
    """register<B> for one peer of a per-rank session."""
    if device is None:
        device = -1
    elif not isinstance(device, int):
        import torch
        device = torch.device(device).index if torch.device(device).index is not None else -1
    c = make_config(device, **cfg)
    return check(library().rc_rank_register(int(rank), int(num_ranks), ctypes.byref(c)))


def rank_finish(rank):
    """finish_collective<B> for one peer; the last one closes the session."""
    return check(library().rc_rank_finish(int(rank)))


def _rank_call(fn, rank, send, recv, op=RC_SUM, root=0, stream=None):
    ref = send if send is not None else recv
    bufs = make_bufs([_ptr(send)], [_ptr(recv)], [tuple(ref.shape)], [_dtype_code(ref)], op, root)
    check(fn(int(rank), ctypes.cast(bufs, ctypes.c_void_p), ctypes.c_void_p(_stream(stream, ref))))


def rank_all_reduce(rank, x, op="sum", out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    _expect(out, x, x.numel(), "rank_all_reduce")
    _rank_call(library().rc_rank_all_reduce, rank, x, out, _op(op), 0, stream)
    return out


def rank_reduce(rank, x, root, op="sum", out=None, stream=None):
    """root counts within rank's communicator (an endpoint's low part)."""
    torch = _torch()
    if out is None and int(rank) % RC_MAX_RANKS == root:
        out = torch.empty_like(x)
    if out is not None and int(rank) % RC_MAX_RANKS == root:
        _expect(out, x, x.numel(), "rank_reduce root")
    _rank_call(library().rc_rank_reduce, rank, x, out, _op(op), root, stream)
    return out


def rank_broadcast(rank, x=None, out=None, stream=None, root=-1):
    """The sender passes x; receivers pass x=None and an `out` tensor (its
    size and dtype are checked against the sender's by the library only
    through the shapes the ranks pass, which must agree)."""
    _rank_call(library().rc_rank_broadcast, rank, x, out, RC_SUM, root, stream)
    return out


def rank_reduce_scatter(rank, x, num_ranks, op="sum", out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(x.numel() // num_ranks, dtype=x.dtype, device=x.device)
    if x.numel() % num_ranks == 0:
        _expect(out, x, x.numel() // num_ranks, "rank_reduce_scatter")
    _rank_call(library().rc_rank_reduce_scatter, rank, x, out, _op(op), 0, stream)
    return out


def rank_all_gather(rank, shard, num_ranks, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(num_ranks * shard.numel(), dtype=shard.dtype, device=shard.device)
    _expect(out, shard, num_ranks * shard.numel(), "rank_all_gather")
    _rank_call(library().rc_rank_all_gather, rank, shard, out, RC_SUM, 0, stream)
    return out


def rank_all_reduce_params(rank, grads, op="mean", out=None, stream=None, acc=None):
    """Rank `rank`'s side of all_reduce_params: its own map {id: tensor}, and
    optionally its map of accumulated gradients."""
    torch = _torch()
    if out is None:
        out = {k: torch.empty_like(v) for k, v in grads.items()}
    n, arr = _param_entries(grads, out, _op(op), acc)
    s = _stream_for(stream, _first_tensor([grads]))
    check(library().rc_rank_all_reduce_params(int(rank), n, ctypes.addressof(arr), ctypes.c_void_p(s)))
    return out


def rank_all_gather_list(rank, shard, num_ranks, out=None, stream=None):
    """Rank `rank`'s side of all_gather_list: out[k] receives rank k's shard."""
    torch = _torch()
    if out is None:
        out = [torch.empty_like(shard) for _ in range(num_ranks)]
    _expect_list(out, num_ranks, "rank_all_gather_list")
    for k, o in enumerate(out):
        _expect(o, shard, shard.numel(), f"rank_all_gather_list output {k}")
    bufs = make_bufs([_ptr(shard)], [None], [tuple(shard.shape)], [_dtype_code(shard)])
    recvs = (ctypes.c_void_p * num_ranks)(*[_ptr(o) for o in out])
    check(library().rc_rank_all_gather_list(int(rank), ctypes.cast(bufs, ctypes.c_void_p), recvs,
                                            ctypes.c_void_p(_stream(stream, shard))))
    return out


def rank_all_to_all_single(rank, x, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    _expect(out, x, x.numel(), "rank_all_to_all_single")
    _rank_call(library().rc_rank_all_to_all_single, rank, x, out, RC_SUM, 0, stream)
    return out


def rank_send(rank, x, dst, stream=None):
    """Communicator.send from logical rank `rank` to `dst`; blocks until dst's
    matching recv arrives."""
    bufs = make_bufs([_ptr(x)], [None], [tuple(x.shape)], [_dtype_code(x)])
    check(library().rc_rank_send(int(rank), ctypes.cast(bufs, ctypes.c_void_p), int(dst),
                                 ctypes.c_void_p(_stream(stream, x))))


def rank_recv(rank, out, src, stream=None):
    """Communicator.recv on logical rank `rank` from `src` into out."""
    bufs = make_bufs([None], [_ptr(out)], [tuple(out.shape)], [_dtype_code(out)])
    check(library().rc_rank_recv(int(rank), ctypes.cast(bufs, ctypes.c_void_p), int(src),
                                 ctypes.c_void_p(_stream(stream, out))))
    return out


def rank_barrier(rank, stream=None):
    """Communicator.barrier for logical rank `rank`."""
    if stream is None:
        s = _torch().cuda.current_stream().cuda_stream
    else:
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    check(library().rc_rank_barrier(int(rank), ctypes.c_void_p(s)))


def rank_split(rank, members):
    """Communicator.split_from for logical rank `rank` (an endpoint): members
    lists the ranks of rank's communicator that form the new one, in order;
    a rank that passes an empty list stays out.  Returns the rank's endpoint
    in the new communicator, or None when it is not a member."""
    members = [int(m) for m in members]
    arr = (ctypes.c_int * max(len(members), 1))(*members)
    out = ctypes.c_int(-1)
    check(library().rc_rank_split(int(rank), len(members), arr, ctypes.byref(out)))
    return out.value if out.value >= 0 else None


def rank_split_all(rank, size):
    """Communicator.split_all: a new communicator of the same `size` ranks."""
    return rank_split(rank, range(size))


class Communicator:
    """One logical rank's communicator, with the method set of the monarch
    `Struct Communicator` page: created once per rank (from that rank's own
    thread), collectives in place on that rank's tensor, a stream per call,
    split_all / split_from for sub-communicators.  Argument marshalling over
    the rank_* functions; errors raise CollectiveError."""

    def __init__(self, rank, world_size, device=None, **cfg):
        rank_register(rank, world_size, device, **cfg)
        self._ep, self._size = int(rank), int(world_size)

    @classmethod
    def _from_endpoint(cls, endpoint, size):
        c = cls.__new__(cls)
        c._ep, c._size = endpoint, size
        return c

    @property
    def rank(self):
        """This rank's index within the communicator."""
        return self._ep % RC_MAX_RANKS

    @property
    def world_size(self):
        return self._size

    def split_all(self):
        """A new communicator of the same ranks (collective over this one)."""
        return Communicator._from_endpoint(rank_split_all(self._ep, self._size), self._size)

    def split_from(self, ranks):
        """A new communicator of `ranks` (in that order); None for a rank left
        out, which may pass an empty list."""
        ranks = list(ranks)
        ep = rank_split(self._ep, ranks)
        return None if ep is None else Communicator._from_endpoint(ep, len(ranks))

    def all_reduce(self, tensor, op="sum", stream=None):
        """Reduce across all ranks, the result in place on every rank."""
        rank_all_reduce(self._ep, tensor, op, out=tensor, stream=stream)

    def broadcast(self, tensor, root, stream=None):
        """The root's tensor to every other rank's tensor."""
        if self.rank == root:
            rank_broadcast(self._ep, tensor, None, stream=stream, root=root)
        else:
            rank_broadcast(self._ep, None, tensor, stream=stream, root=root)

    def reduce(self, tensor, op, root, stream=None):
        """Reduce across all ranks into the root's tensor (in place)."""
        rank_reduce(self._ep, tensor, root, op, out=tensor if self.rank == root else None, stream=stream)

    def all_gather(self, output_tensors, input_tensor, stream=None):
        """Every rank's input into this rank's list of outputs, one per rank."""
        rank_all_gather_list(self._ep, input_tensor, self._size, out=list(output_tensors), stream=stream)

    def all_gather_into_tensor(self, output, input, stream=None):
        rank_all_gather(self._ep, input, self._size, out=output, stream=stream)

    def reduce_scatter_tensor(self, output, input, op="sum", stream=None):
        rank_reduce_scatter(self._ep, input, self._size, op, out=output, stream=stream)

    def send(self, tensor, dst, stream=None):
        rank_send(self._ep, tensor, dst, stream=stream)

    def recv(self, tensor, src, stream=None):
        rank_recv(self._ep, tensor, src, stream=stream)

    def all_to_all_single(self, output, input, stream=None):
        rank_all_to_all_single(self._ep, input, out=output, stream=stream)

    def barrier(self, stream=None):
        rank_barrier(self._ep, stream=stream)

    def all_reduce_params(self, grads, op="mean", out=None, stream=None, acc=None):
        """The gradient sync keyed by parameter ID for this rank's map."""
        return rank_all_reduce_params(self._ep, grads, op, out=out, stream=stream, acc=acc)

    def finish(self):
        rank_finish(self._ep)
