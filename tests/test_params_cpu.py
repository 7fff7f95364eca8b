"""The parameter-keyed gradient sync on the CPU (validate-only sessions, fake
addresses): entries pair by ID in any order, and every ID, dtype, shape and
argument error comes back with its code, from the whole-call and the
per-rank entry points."""

import ctypes
import random
import threading

import pytest

import rank_reductions_amd as rr

MiB = 1 << 20
# parameter id -> shape; shapes differ per ID, so pairing by position fails
SPECS = {11: (4, 8), 3: (257,), 40: (0,), 7: (), 2: (3, 3, 3), 99: (1024,)}


@pytest.fixture
def lib():
    lib = rr.library()
    lib.rc_reset()
    yield lib
    lib.rc_reset()


def cfg():
    return rr.make_config(validate_only=True)


def rank_entries(r, specs=SPECS, order_seed=None, dtype=rr.RC_F32, op=rr.RC_MEAN, edits=None, accs=None):
    """(count, rc_param array) of rank r: each parameter at its own fake
    send/recv range, listed in a per-rank shuffled order; accs maps an ID to
    its accumulator address."""
    keys = list(specs)
    random.Random(order_seed if order_seed is not None else r).shuffle(keys)
    shapes, sends, recvs, dts, ops = [], [], [], [], []
    for k in keys:
        shapes.append(specs[k])
        sends.append(0x100000000 + r * 256 * MiB + k * MiB)
        recvs.append(0x800000000 + r * 256 * MiB + k * MiB)
        dts.append(dtype)
        ops.append(op)
    if edits:
        edits(keys, shapes, sends, recvs, dts, ops)
    n = len(keys)
    arr = (rr.RcParam * max(n, 1))()
    if n:
        bufs = rr.make_bufs(sends, recvs, shapes, dts, ops)
        for i, k in enumerate(keys):
            arr[i].id = k
            arr[i].buf = bufs[i]
            arr[i].acc = (accs or {}).get(k)
    return n, arr


def acc_addr(r, k):
    return 0x1000000000 + r * 256 * MiB + k * MiB


def whole_call(lib, entries):
    R = len(entries)
    counts = (ctypes.c_int * R)(*[e[0] for e in entries])
    params = (ctypes.c_void_p * R)(*[ctypes.addressof(e[1]) for e in entries])
    code = lib.rc_all_reduce_params(counts, params, None)
    return code, lib.rc_last_error().decode()


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_shuffled_orders_pair_by_id(lib, R):
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    code, msg = whole_call(lib, [rank_entries(r) for r in range(R)])
    assert code == rr.RC_OK, msg


def test_id_sets_must_agree(lib):
    R = 3
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    missing = {k: v for k, v in SPECS.items() if k != 40}
    code, msg = whole_call(lib, [rank_entries(0), rank_entries(1, missing), rank_entries(2)])
    assert code == rr.RC_ERR_PARAM_MISMATCH and "parameter 40" in msg and "rank 1" in msg, msg
    extra = {**SPECS, 5: (2,)}
    code, msg = whole_call(lib, [rank_entries(0), rank_entries(1), rank_entries(2, extra)])
    assert code == rr.RC_ERR_PARAM_MISMATCH and "parameter 5" in msg, msg
    renamed = {(12 if k == 11 else k): v for k, v in SPECS.items()}
    code, msg = whole_call(lib, [rank_entries(0), rank_entries(1, renamed), rank_entries(2)])
    assert code == rr.RC_ERR_PARAM_MISMATCH and "parameter 11" in msg, msg
    # the ID check comes before any per-parameter check
    def bad_shape(keys, shapes, *_):
        shapes[0] = (5,)
    code, msg = whole_call(lib, [rank_entries(0, missing, edits=bad_shape), rank_entries(1), rank_entries(2)])
    assert code == rr.RC_ERR_PARAM_MISMATCH, msg


def test_per_parameter_checks_name_the_id(lib):
    R = 2
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK

    def shape_of_99(keys, shapes, *_):
        shapes[keys.index(99)] = (1023,)
    code, msg = whole_call(lib, [rank_entries(0), rank_entries(1, edits=shape_of_99)])
    assert code == rr.RC_ERR_SHAPE_MISMATCH and "parameter 99" in msg, msg

    def dtype_of_3(keys, shapes, sends, recvs, dts, ops):
        dts[keys.index(3)] = rr.RC_I32
    code, msg = whole_call(lib, [rank_entries(0, edits=dtype_of_3), rank_entries(1)])
    assert code == rr.RC_ERR_DTYPE_MISMATCH and "parameter 3" in msg, msg

    def null_send_of_7(keys, shapes, sends, *_):
        sends[keys.index(7)] = None
    code, msg = whole_call(lib, [rank_entries(0), rank_entries(1, edits=null_send_of_7)])
    assert code == rr.RC_ERR_INVALID_ARGUMENT and "parameter 7" in msg, msg

    def op_sum(keys, shapes, sends, recvs, dts, ops):
        ops[:] = [rr.RC_SUM] * len(ops)
    code, msg = whole_call(lib, [rank_entries(0, edits=op_sum), rank_entries(1, edits=op_sum)])
    assert code == rr.RC_OK, msg
    code, msg = whole_call(lib, [rank_entries(0, edits=op_sum), rank_entries(1)])
    assert code == rr.RC_ERR_OP_MISMATCH, msg

    def overlapping_outputs(keys, shapes, sends, recvs, *_):
        recvs[keys.index(2)] = recvs[keys.index(99)] + 64
    code, msg = whole_call(lib, [rank_entries(0, edits=overlapping_outputs), rank_entries(1)])
    assert code == rr.RC_ERR_INVALID_ARGUMENT, msg


def test_argument_errors(lib):
    R = 2
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK

    def dup(keys, shapes, sends, recvs, dts, ops):
        keys.append(keys[0])
        shapes.append(shapes[0])
        sends.append(sends[0] + 128 * MiB)
        recvs.append(recvs[0] + 128 * MiB)
        dts.append(dts[0])
        ops.append(ops[0])
    code, msg = whole_call(lib, [rank_entries(0, edits=dup), rank_entries(1)])
    assert code == rr.RC_ERR_INVALID_ARGUMENT and "twice" in msg, msg
    e0 = rank_entries(0)
    counts = (ctypes.c_int * R)(-1, e0[0])
    params = (ctypes.c_void_p * R)(ctypes.addressof(e0[1]), ctypes.addressof(e0[1]))
    assert lib.rc_all_reduce_params(counts, params, None) == rr.RC_ERR_INVALID_ARGUMENT
    counts = (ctypes.c_int * R)(e0[0], e0[0])
    params = (ctypes.c_void_p * R)(ctypes.addressof(e0[1]), None)
    assert lib.rc_all_reduce_params(counts, params, None) == rr.RC_ERR_INVALID_ARGUMENT
    assert lib.rc_all_reduce_params(None, params, None) == rr.RC_ERR_INVALID_ARGUMENT
    assert lib.rc_all_reduce_params(counts, None, None) == rr.RC_ERR_INVALID_ARGUMENT
    # nothing to sync is fine
    code, msg = whole_call(lib, [rank_entries(0, {}), rank_entries(1, {})])
    assert code == rr.RC_OK, msg
    # and a session opened per rank refuses the whole-call form
    lib.rc_reset()
    assert lib.rc_rank_register(0, R, ctypes.byref(cfg())) == rr.RC_OK
    code, _ = whole_call(lib, [rank_entries(0), rank_entries(1)])
    assert code == rr.RC_ERR_INVALID_ARGUMENT


def test_unregistered(lib):
    code, _ = whole_call(lib, [rank_entries(0)])
    assert code == rr.RC_ERR_NOT_REGISTERED


def run_ranks(R, body):
    out = [None] * R
    errs = []

    def go(r):
        try:
            out[r] = body(r)
        except BaseException as e:  # noqa: BLE001
            errs.append(e)

    ts = [threading.Thread(target=go, args=(r,)) for r in range(R)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert not errs, errs
    assert all(not t.is_alive() for t in ts)
    return out


def rank_params(lib, r, entry):
    n, arr = entry
    return lib.rc_rank_all_reduce_params(r, n, ctypes.addressof(arr), None)


def test_per_rank_sync(lib):
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        res = []
        for it in range(20):
            res.append(rank_params(lib, r, rank_entries(r, order_seed=100 * it + r)))
        missing = {k: v for k, v in SPECS.items() if k != 2} if r == 3 else SPECS
        res.append(rank_params(lib, r, rank_entries(r, missing)))
        if r == 1:
            b = rr.make_bufs([0x100000000 + r * 256 * MiB], [0x800000000 + r * 256 * MiB], (8,))
            res.append(lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None))
        else:
            res.append(rank_params(lib, r, rank_entries(r)))
        if r == 2:
            res.append(lib.rc_rank_all_reduce_params(r, 3, None, None))
        else:
            res.append(rank_params(lib, r, rank_entries(r)))
        res.append(rank_params(lib, r, rank_entries(r)))
        res.append(lib.rc_rank_finish(r))
        return res

    for res in run_ranks(R, body):
        assert res[:20] == [rr.RC_OK] * 20
        assert res[20] == rr.RC_ERR_PARAM_MISMATCH
        assert res[21] == rr.RC_ERR_OP_MISMATCH
        assert res[22] == rr.RC_ERR_INVALID_ARGUMENT
        assert res[23] == rr.RC_OK
        assert res[24] == rr.RC_OK


def test_accumulators(lib):
    """acc on every rank or none, Sum/Mean only, aligned, and overlapping
    nothing but its own rank's output."""
    R = 3
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    every = [rank_entries(r, accs={k: acc_addr(r, k) for k in SPECS}) for r in range(R)]
    code, msg = whole_call(lib, every)
    assert code == rr.RC_OK, msg
    # only some parameters carry accumulators: fine, they are batched apart
    some = [rank_entries(r, accs={k: acc_addr(r, k) for k in (3, 99)}) for r in range(R)]
    code, msg = whole_call(lib, some)
    assert code == rr.RC_OK, msg
    partial = [rank_entries(r, accs={99: acc_addr(r, 99)} if r != 1 else {}) for r in range(R)]
    code, msg = whole_call(lib, partial)
    assert code == rr.RC_ERR_INVALID_ARGUMENT and "parameter 99" in msg and "some ranks" in msg, msg
    mx = [rank_entries(r, op=rr.RC_MAX, accs={3: acc_addr(r, 3)}) for r in range(R)]
    code, msg = whole_call(lib, mx)
    assert code == rr.RC_ERR_INVALID_ARGUMENT and "Sum or Mean" in msg, msg
    mis = [rank_entries(r, accs={3: acc_addr(r, 3) + (2 if r == 2 else 0)}) for r in range(R)]
    code, msg = whole_call(lib, mis)
    assert code == rr.RC_ERR_INVALID_ARGUMENT and "misaligned" in msg, msg
    # in place into the accumulator: recv == acc on every rank
    def recv_is_acc(r):
        def edit(keys, shapes, sends, recvs, dts, ops):
            recvs[keys.index(99)] = acc_addr(r, 99)
        return edit
    inplace = [rank_entries(r, edits=recv_is_acc(r), accs={99: acc_addr(r, 99)}) for r in range(R)]
    code, msg = whole_call(lib, inplace)
    assert code == rr.RC_OK, msg
    # an accumulator that is another rank's output
    clash = [rank_entries(r, accs={99: (0x800000000 + 256 * MiB + 99 * MiB) if r == 0 else acc_addr(r, 99)})
             for r in range(R)]
    code, msg = whole_call(lib, clash)
    assert code == rr.RC_ERR_INVALID_ARGUMENT, msg
    # and an empty parameter ignores its accumulator fields entirely
    empty = [rank_entries(r, accs={40: acc_addr(r, 40)} if r == 0 else {}) for r in range(R)]
    code, msg = whole_call(lib, empty)
    assert code == rr.RC_OK, msg
