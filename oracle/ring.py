"""Plain CPU oracle for collectives over R logical ranks.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

What it computes, and where that is defined
-------------------------------------------
* ruCCL README (ja), "CUDA tensor example" and user guide section 5 "CUDA
  example": several logical ranks on one GPU run a *ring* AllReduce and check
  the sum / mean of FP32 elements, with the original inputs left unchanged.
* ruCCL README (ja), user guide section 2 "Tensor collective API": all_reduce
  returns the reduced result to every participant; broadcast has one sender
  (Some(tensor)) and receivers that pass nothing; reduce delivers to one root
  and non-root participants receive nothing.
* monarch `Struct Communicator` page, methods `reduce_scatter_tensor` ("reduce,
  then scatter the result"), `all_gather_into_tensor` (gather every rank's
  tensor into one output), and `all_reduce` (result in place on every rank).
* RUDA "Training and state saving", section "Configure training backend": the
  backend element types are f32 and i32, so the dtypes here are float32 and
  int32 and all float arithmetic is float32 (the pages fix that precision).
* ruCCL README (ja), section 6 "Collective training": the whole gradient set,
  keyed by parameter ID, is reduced with Mean; IDs, shapes and dtype must
  agree on every rank.  RUDA "Training and state saving", gradient
  accumulation: accumulate adds without averaging.

Readings where the pages are silent (each restated where it is used):
* Segments: S = ceil(N / R); segment c is [c*S, min((c+1)*S, N)), possibly
  empty.
* Ring: rank r sends to rank (r + 1) mod R.  Reduce-scatter step s (0..R-2):
  rank r passes its partial of segment (r - s - 1) mod R to rank r + 1, which
  combines it with its own input of that segment.  Segment c therefore ends at
  its owner c, folded left in rank order (c+1), (c+2), ..., c.
* Mean is one correctly rounded float32 division of the finished fold by R,
  done by the owner before the all-gather.  int32 Mean is not defined.
* int32 Sum wraps (two's complement); int32 Max is the ordinary maximum.
* float32 Max: if any operand is NaN the result is the canonical quiet NaN
  0x7FC00000; otherwise the larger value, with +0 counted above -0.
* All-gather step s (0..R-2): rank r passes finished segment (r - s) mod R to
  rank r + 1, which copies it bit for bit.

Everything operates on NumPy arrays on the host.  Float arithmetic is float32
elementwise (each add is one IEEE round-to-nearest-even operation, subnormals
kept); nothing is blocked, fused or reordered beyond the ring steps above.
"""

import numpy as np

SUM = "sum"
MEAN = "mean"
MAX = "max"
OPS = (SUM, MEAN, MAX)

CANONICAL_NAN_BITS = np.uint32(0x7FC00000)


class OracleError(ValueError):
    """Raised for calls the pages declare invalid (e.g. two broadcast senders)."""


# --------------------------------------------------------------------------
# Elementwise operators
# --------------------------------------------------------------------------

def _check_dtype(a):
    if a.dtype not in (np.float32, np.int32):
        raise OracleError(f"unsupported dtype {a.dtype}; the backend types are f32 and i32")


def combine(a, b, op):
    """One reduction step a (+) b, elementwise, in the arrays' own dtype.

    Sum and Mean fold with '+' (ruCCL README, section 2: all_reduce returns
    the reduced result; the example checks sum and mean).  Max follows the
    ReduceOp of the monarch Communicator page's all_reduce.
    """
    _check_dtype(a)
    if a.dtype != b.dtype:
        raise OracleError("dtype mismatch between ranks")
    if op in (SUM, MEAN):
        if a.dtype == np.int32:
            # two's-complement wrap, written out explicitly
            wide = a.astype(np.int64) + b.astype(np.int64)
            return (wide & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        return np.add(a, b, dtype=np.float32)
    if op == MAX:
        if a.dtype == np.int32:
            return np.maximum(a, b)
        return _max_f32(a, b)
    raise OracleError(f"unknown op {op!r}")


def _max_f32(a, b):
    """float32 max: NaN wins (as the canonical quiet NaN); +0 beats -0."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    out = np.where(a > b, a, b).astype(np.float32)
    # the only pair that compares equal with different bits is (+0, -0)
    both_zero = (a == 0) & (b == 0)
    both_negative = np.signbit(a) & np.signbit(b)
    signed_zero = np.where(both_negative, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    out = np.where(both_zero, signed_zero, out).astype(np.float32)
    bits = out.view(np.uint32).copy()
    bits[np.isnan(a) | np.isnan(b)] = CANONICAL_NAN_BITS
    return bits.view(np.float32)


def finish(acc, op, num_ranks):
    """Applied once to a finished fold: Mean divides by R (float32, rounded once)."""
    if op == MEAN:
        if acc.dtype != np.float32:
            raise OracleError("Mean is defined for float32 only")
        return np.divide(acc, np.float32(num_ranks), dtype=np.float32)
    return acc


# --------------------------------------------------------------------------
# Segmentation
# --------------------------------------------------------------------------

def segment_length(n, num_ranks):
    """S = ceil(N / R), the ring segment length (reading: the pages name a ring
    AllReduce but print no chunking rule)."""
    if num_ranks <= 0:
        raise OracleError("need at least one rank")
    return -(-n // num_ranks)


def segment_bounds(n, num_ranks):
    """[(start, end)] of the R ring segments; trailing segments may be empty."""
    s = segment_length(n, num_ranks)
    return [(min(c * s, n), min((c + 1) * s, n)) for c in range(num_ranks)]


def _validate_ranks(xs, same_shape=True):
    if len(xs) == 0:
        raise OracleError("need at least one rank")
    for x in xs:
        _check_dtype(np.asarray(x))
    if any(np.asarray(x).dtype != np.asarray(xs[0]).dtype for x in xs):
        raise OracleError("dtype mismatch between ranks")
    if same_shape and any(np.shape(x) != np.shape(xs[0]) for x in xs):
        raise OracleError("shape mismatch between ranks")


def _flat(x):
    return np.ascontiguousarray(x).reshape(-1)


# --------------------------------------------------------------------------
# The ring, step by step
# --------------------------------------------------------------------------

def ring_reduce_scatter_phase(xs, op):
    """Reduce-scatter phase of the ring AllReduce, simulated message by message.

    Returns (state, bounds): state[r] is rank r's working buffer after R-1
    steps; the finished (and, for Mean, divided) segment c sits in state[c].
    """
    R = len(xs)
    flat = [_flat(x) for x in xs]
    n = flat[0].size
    bounds = segment_bounds(n, R)
    state = [x.copy() for x in flat]
    for s in range(R - 1):
        # every rank sends at once; collect the messages before applying them
        messages = []
        for r in range(R):
            c = (r - s - 1) % R
            lo, hi = bounds[c]
            messages.append(((r + 1) % R, c, state[r][lo:hi].copy()))
        for dst, c, received in messages:
            lo, hi = bounds[c]
            state[dst][lo:hi] = combine(received, flat[dst][lo:hi], op)
    for c in range(R):
        lo, hi = bounds[c]
        state[c][lo:hi] = finish(state[c][lo:hi], op, R)
    return state, bounds


def ring_all_gather_phase(state, bounds):
    """All-gather phase: finished segments travel the ring and are copied."""
    R = len(state)
    for s in range(R - 1):
        messages = []
        for r in range(R):
            c = (r - s) % R
            lo, hi = bounds[c]
            messages.append(((r + 1) % R, c, state[r][lo:hi].copy()))
        for dst, c, received in messages:
            lo, hi = bounds[c]
            state[dst][lo:hi] = received
    return state


def all_reduce(xs, op=SUM):
    """Ring AllReduce (ruCCL README, "CUDA tensor example"): every rank gets the
    reduced result; the inputs are not modified.  Returns R arrays shaped like
    the inputs."""
    _validate_ranks(xs)
    shape = np.shape(xs[0])
    state, bounds = ring_reduce_scatter_phase(xs, op)
    state = ring_all_gather_phase(state, bounds)
    return [s.reshape(shape) for s in state]


def reduce(xs, root, op=SUM):
    """reduce to a root (ruCCL README section 2; monarch Communicator.reduce):
    the root receives the reduction, every other rank receives nothing (None).

    Reading: the reduce-scatter phase runs as in all_reduce and the root then
    collects each owner's finished segment, so the root's bits equal
    all_reduce's."""
    _validate_ranks(xs)
    R = len(xs)
    if not 0 <= root < R:
        raise OracleError("root out of range")
    shape = np.shape(xs[0])
    state, bounds = ring_reduce_scatter_phase(xs, op)
    result = np.empty_like(state[0])
    for c, (lo, hi) in enumerate(bounds):
        result[lo:hi] = state[c][lo:hi]
    out = [None] * R
    out[root] = result.reshape(shape)
    return out


def broadcast(sends):
    """broadcast (ruCCL README section 2): exactly one rank passes a tensor,
    the others pass None; every rank receives the sender's bytes.  Any other
    sender count is an error (section 4, CollectiveError)."""
    senders = [i for i, x in enumerate(sends) if x is not None]
    if len(senders) != 1:
        raise OracleError(f"broadcast needs exactly one sender, got {len(senders)}")
    src = np.ascontiguousarray(sends[senders[0]])
    _check_dtype(src)
    R = len(sends)
    # along the ring from the sender: each hop copies what it received
    out = [None] * R
    out[senders[0]] = src.copy()
    for hop in range(1, R):
        prev = (senders[0] + hop - 1) % R
        out[(senders[0] + hop) % R] = out[prev].copy()
    return out


def reduce_scatter(xs, op=SUM):
    """reduce_scatter_tensor (monarch Communicator page): reduce, then scatter.
    Each rank's input holds R*M elements; rank r receives the M-element shard
    [r*M, (r+1)*M) of the reduction.  N not divisible by R is an error."""
    _validate_ranks(xs)
    R = len(xs)
    n = _flat(xs[0]).size
    if n % R:
        raise OracleError("reduce_scatter input length must be a multiple of R")
    state, bounds = ring_reduce_scatter_phase(xs, op)
    return [state[r][lo:hi].copy() for r, (lo, hi) in enumerate(bounds)]


def all_gather(shards):
    """all_gather_into_tensor (monarch Communicator page): every rank receives
    the concatenation shard_0, ..., shard_{R-1}, bit for bit."""
    _validate_ranks(shards)
    R = len(shards)
    flat = [_flat(x) for x in shards]
    m = flat[0].size
    state = [np.zeros(R * m, dtype=flat[0].dtype) for _ in range(R)]
    bounds = [(k * m, (k + 1) * m) for k in range(R)]
    for r in range(R):
        lo, hi = bounds[r]
        state[r][lo:hi] = flat[r]
    return ring_all_gather_phase(state, bounds)


def all_reduce_many(tensors, op=MEAN):
    """Whole-gradient reduction (ruCCL README section 6, "Collective training":
    the gradients are reduced with ReduceOperation::Mean).  tensors[t][r] is
    rank r's copy of tensor t; each tensor is reduced on its own, with its own
    ring segments.  Returns out[t][r]."""
    return [all_reduce(list(per_rank), op) for per_rank in tensors]


# --------------------------------------------------------------------------
# Copies between ranks (monarch Communicator page)
# --------------------------------------------------------------------------

def all_gather_list(shards):
    """Communicator.all_gather, the list form: every rank receives one output
    tensor per source rank, the k-th being rank k's input.  Returns out[r][k]
    (copies)."""
    _validate_ranks(shards)
    R = len(shards)
    return [[np.array(shards[k], copy=True) for k in range(R)] for _ in range(R)]


def all_to_all_single(xs):
    """Communicator.all_to_all_single: each rank's input is split into R equal
    chunks, chunk d is scattered to rank d, and each rank concatenates the
    chunks it receives in source-rank order.  An input length not divisible by
    R is an error (the page's form has no split sizes, so the chunks are
    equal).  Returns R arrays shaped like the inputs."""
    _validate_ranks(xs)
    R = len(xs)
    shape = np.shape(xs[0])
    flat = [_flat(x) for x in xs]
    n = flat[0].size
    if n % R:
        raise OracleError("all_to_all_single input length must be a multiple of R")
    m = n // R
    out = [np.empty_like(flat[0]) for _ in range(R)]
    for src in range(R):
        for dst in range(R):
            out[dst][src * m:(src + 1) * m] = flat[src][dst * m:(dst + 1) * m]
    return [o.reshape(shape) for o in out]


def send_recv(x):
    """Communicator.send on the source rank and recv on the destination: the
    receiver's tensor gets the sender's bytes."""
    x = np.asarray(x)
    _check_dtype(x)
    return x.copy()


# --------------------------------------------------------------------------
# Gradient synchronisation keyed by parameter ID
# --------------------------------------------------------------------------

class ParamMismatch(OracleError):
    """The ranks' gradient maps disagree.  kind is "ids" (the ID sets differ),
    "dtype" or "shape" (one ID's tensors differ between ranks)."""

    def __init__(self, kind, msg):
        super().__init__(msg)
        self.kind = kind


def all_reduce_params(grads, op=MEAN, acc=None):
    """Whole-gradient sync of ruCCL README section 6, "Collective training":
    every rank holds a map from parameter ID to gradient and reduces it with
    ReduceOperation::Mean; the IDs, each gradient's shape and the dtype must
    agree on every rank.

    grads[r] is rank r's map {id: array}.  Readings: entries are paired across
    ranks by ID (a map has no order, so the order a rank lists its entries in
    does not matter); each parameter is reduced on its own, exactly as one
    all_reduce of that parameter's R tensors; mismatches are checked IDs
    first, then per parameter (in ID order) dtype before shape.  Returns R
    maps {id: reduced array}, every rank's values identical.

    acc, if given, is one map per rank of accumulated gradients (RUDA
    "Training and state saving": the accumulator sums microbatch gradients
    and hands the sum to the sync).  A parameter with an accumulator is
    reduced over accumulate(acc, grad), the last microbatch added first.
    Readings: a non-empty parameter has an accumulator on every rank or on
    none; accumulated gradients are reduced with Sum or Mean only."""
    R = len(grads)
    if R == 0:
        raise OracleError("need at least one rank")
    ids = set(grads[0])
    for r in range(1, R):
        if set(grads[r]) != ids:
            only0 = sorted(ids - set(grads[r]))
            onlyr = sorted(set(grads[r]) - ids)
            raise ParamMismatch("ids", f"rank {r}: missing {only0[:3]}, extra {onlyr[:3]}")
    for pid in sorted(ids):
        per_rank = [np.asarray(grads[r][pid]) for r in range(R)]
        if any(a.dtype != per_rank[0].dtype for a in per_rank):
            raise ParamMismatch("dtype", f"parameter {pid}: dtype differs between ranks")
        if any(a.shape != per_rank[0].shape for a in per_rank):
            raise ParamMismatch("shape", f"parameter {pid}: shape differs between ranks")
    out = [{} for _ in range(R)]
    for pid in ids:
        operands = [grads[r][pid] for r in range(R)]
        if acc is not None and np.asarray(operands[0]).size:
            given = [pid in acc[r] for r in range(R)]
            if any(given) and not all(given):
                raise OracleError(f"parameter {pid}: accumulator on some ranks only")
            if all(given):
                if op == MAX:
                    raise OracleError(f"parameter {pid}: accumulated gradients reduce with Sum or Mean")
                operands = [accumulate(acc[r][pid], operands[r]) for r in range(R)]
        reduced = all_reduce(operands, op)
        for r in range(R):
            out[r][pid] = reduced[r]
    return out


def accumulate(acc, grad):
    """GradientsAccumulator.accumulate (RUDA "Training and state saving",
    gradient accumulation): gradients are added without averaging.  acc is None
    for an empty accumulator, which then takes a copy of grad.  One float32
    add per element (int32 wraps)."""
    grad = np.asarray(grad)
    _check_dtype(grad)
    if acc is None:
        return grad.copy()
    acc = np.asarray(acc)
    if acc.dtype != grad.dtype or acc.shape != grad.shape:
        raise OracleError("accumulate: dtype or shape differs from the accumulator")
    return combine(_flat(acc), _flat(grad), SUM).reshape(acc.shape)


# --------------------------------------------------------------------------
# Closed form of the ring order, and single elements of it
# --------------------------------------------------------------------------

def fold_order(c, num_ranks):
    """Rank order in which segment c is folded: (c+1), (c+2), ..., c  (mod R)."""
    return [(c + k) % num_ranks for k in range(1, num_ranks + 1)]


def all_reduce_closed_form(xs, op=SUM):
    """The result the ring leaves on every rank, computed segment by segment as
    a left fold in the order fold_order(c).  One array, shaped like the input."""
    _validate_ranks(xs)
    R = len(xs)
    flat = [_flat(x) for x in xs]
    out = np.empty_like(flat[0])
    for c, (lo, hi) in enumerate(segment_bounds(flat[0].size, R)):
        order = fold_order(c, R)
        acc = flat[order[0]][lo:hi].copy()
        for r in order[1:]:
            acc = combine(acc, flat[r][lo:hi], op)
        out[lo:hi] = finish(acc, op, R)
    return out.reshape(np.shape(xs[0]))


def all_reduce_at(values, index, n, op=SUM):
    """The all_reduce result at one element index, from that element's value on
    each rank (values[r]).  Used to check sampled outputs of very large calls."""
    values = np.asarray(values)
    R = values.shape[0]
    c = index // segment_length(n, R)
    order = fold_order(c, R)
    acc = values[order[0]:order[0] + 1].copy()
    for r in order[1:]:
        acc = combine(acc, values[r:r + 1], op)
    return finish(acc, op, R)[0]


def all_reduce_at_many(values, indices, n, op=SUM):
    """Vector form of all_reduce_at: values is [R, K] (rank r's value at each of
    K sampled indices), indices is [K].  Elements are grouped by segment so each
    group is folded in its own order."""
    values = np.asarray(values)
    indices = np.asarray(indices, dtype=np.int64)
    R = values.shape[0]
    s = segment_length(n, R)
    seg = indices // s
    out = np.empty(values.shape[1], dtype=values.dtype)
    for c in np.unique(seg):
        sel = seg == c
        order = fold_order(int(c), R)
        acc = values[order[0], sel].copy()
        for r in order[1:]:
            acc = combine(acc, values[r, sel], op)
        out[sel] = finish(acc, op, R)
    return out
