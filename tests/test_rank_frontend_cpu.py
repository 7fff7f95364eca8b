"""The per-rank front end on the CPU (validate-only sessions, fake addresses):
one thread per logical rank, calls matched by issue order, mismatches reported
to every rank, registration errors, and reset releasing waiting ranks."""

import ctypes
import threading
import time

import pytest

import rank_reductions_amd as rr

MiB = 1 << 20


@pytest.fixture
def lib():
    lib = rr.library()
    lib.rc_reset()
    yield lib
    lib.rc_reset()


def cfg():
    return rr.make_config(validate_only=True)


def one(send, recv, n=1024, dtype=rr.RC_F32, op=rr.RC_SUM, root=0):
    return rr.make_bufs([send], [recv], (n,), dtype, op, root)


def run_ranks(R, body):
    """Run body(rank) on R threads; returns the per-rank results."""
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
    assert all(not t.is_alive() for t in ts), "a rank thread did not return"
    return out


def send_addr(r):
    return 0x10000000 + r * 4 * MiB


def recv_addr(r):
    return 0x80000000 + r * 4 * MiB


def test_matching_calls_succeed(lib):
    R = 4

    def body(r):
        codes = [lib.rc_rank_register(r, R, ctypes.byref(cfg()))]
        for i in range(30):
            b = one(send_addr(r), recv_addr(r), n=1000 + i)
            fn = (lib.rc_rank_all_reduce, lib.rc_rank_reduce, lib.rc_rank_all_gather)[i % 3]
            codes.append(fn(r, ctypes.cast(b, ctypes.c_void_p), None))
        sends = send_addr(r) if r == 2 else 0
        b = one(sends, recv_addr(r), root=-1)
        codes.append(lib.rc_rank_broadcast(r, ctypes.cast(b, ctypes.c_void_p), None))
        codes.append(lib.rc_rank_finish(r))
        return codes

    for codes in run_ranks(R, body):
        assert codes == [rr.RC_OK] * len(codes)
    # the session closed when the last rank finished
    b = one(send_addr(0), recv_addr(0))
    assert lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_ERR_NOT_REGISTERED


def test_mismatches_reported_to_every_rank(lib):
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        res = []
        b = one(send_addr(r), recv_addr(r), n=1024 if r != 2 else 1000)
        res.append(lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None))
        res.append(lib.rc_last_error().decode())
        b = one(send_addr(r), recv_addr(r), op=rr.RC_MAX if r == 3 else rr.RC_SUM)
        res.append(lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None))
        b = one(send_addr(r), recv_addr(r))
        fn = lib.rc_rank_broadcast if r == 1 else lib.rc_rank_all_reduce
        res.append(fn(r, ctypes.cast(b, ctypes.c_void_p), None))
        b = one(send_addr(r), recv_addr(r), root=1 if r else 0)
        res.append(lib.rc_rank_reduce(r, ctypes.cast(b, ctypes.c_void_p), None))
        b = one(send_addr(r), recv_addr(r))
        res.append(lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None))
        return res

    for res in run_ranks(R, body):
        assert res[0] == rr.RC_ERR_SHAPE_MISMATCH and "rank 2" in res[1]
        assert res[2] == rr.RC_ERR_OP_MISMATCH
        assert res[3] == rr.RC_ERR_OP_MISMATCH       # broadcast against all_reduce
        assert res[4] == rr.RC_ERR_ROOT_MISMATCH
        assert res[5] == rr.RC_OK                     # the session is still usable


def test_registration_errors(lib):
    R = 3
    assert lib.rc_rank_register(0, R, ctypes.byref(cfg())) == rr.RC_OK
    assert lib.rc_rank_register(0, R, ctypes.byref(cfg())) == rr.RC_ERR_DUPLICATE_REGISTRATION
    assert lib.rc_rank_register(1, R + 1, ctypes.byref(cfg())) == rr.RC_ERR_INVALID_ARGUMENT
    assert lib.rc_rank_register(R, R, ctypes.byref(cfg())) == rr.RC_ERR_INVALID_ARGUMENT
    b = one(send_addr(1), recv_addr(1))
    assert lib.rc_rank_all_reduce(1, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_ERR_NOT_REGISTERED
    assert lib.rc_rank_finish(2) == rr.RC_ERR_NOT_REGISTERED
    # the whole-call entry points refuse a per-rank session
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_ERR_DUPLICATE_REGISTRATION
    bufs = rr.make_bufs([send_addr(r) for r in range(R)], [recv_addr(r) for r in range(R)], (8,))
    assert lib.rc_all_reduce(ctypes.cast(bufs, ctypes.c_void_p), None) == rr.RC_ERR_INVALID_ARGUMENT
    assert lib.rc_finish() == rr.RC_ERR_INVALID_ARGUMENT
    lib.rc_reset()
    # and a whole-call session refuses per-rank registration
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    assert lib.rc_rank_register(0, R, ctypes.byref(cfg())) == rr.RC_ERR_DUPLICATE_REGISTRATION
    assert lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_ERR_NOT_REGISTERED


def test_reset_releases_waiting_ranks(lib):
    R = 4
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK

    def body(r):
        if r == R - 1:  # this rank never calls; it resets the session instead
            time.sleep(0.3)
            return lib.rc_reset()
        b = one(send_addr(r), recv_addr(r))
        return lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None)

    res = run_ranks(R, body)
    assert res[:R - 1] == [rr.RC_ERR_NOT_REGISTERED] * (R - 1)
    assert res[R - 1] == rr.RC_OK


def test_null_buf_is_reported_to_all(lib):
    R = 2

    def body(r):
        lib.rc_rank_register(r, R, ctypes.byref(cfg()))
        if r == 1:
            return lib.rc_rank_all_reduce(r, None, None)
        b = one(send_addr(r), recv_addr(r))
        return lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None)

    assert run_ranks(R, body) == [rr.RC_ERR_INVALID_ARGUMENT] * R


def test_second_call_of_a_busy_rank_is_refused(lib):
    R = 2
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
    first = {}

    def rank0():
        b = one(send_addr(0), recv_addr(0))
        first["rc"] = lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None)

    t = threading.Thread(target=rank0)
    t.start()
    time.sleep(0.2)  # rank 0's call is now waiting for rank 1
    b = one(send_addr(0), recv_addr(0))
    assert lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_ERR_INVALID_ARGUMENT
    assert "in progress" in lib.rc_last_error().decode()
    b = one(send_addr(1), recv_addr(1))
    assert lib.rc_rank_all_reduce(1, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_OK
    t.join(timeout=30)
    assert first["rc"] == rr.RC_OK
    # the refused call joined no collective: the next calls still pair up
    res = run_ranks(R, lambda r: lib.rc_rank_all_reduce(
        r, ctypes.cast(one(send_addr(r), recv_addr(r)), ctypes.c_void_p), None))
    assert res == [rr.RC_OK] * R


def test_finish_refused_while_the_rank_waits(lib):
    R = 2
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
    first = {}

    def rank0():
        b = one(send_addr(0), recv_addr(0))
        first["rc"] = lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None)

    t = threading.Thread(target=rank0)
    t.start()
    time.sleep(0.2)
    assert lib.rc_rank_finish(0) == rr.RC_ERR_INVALID_ARGUMENT
    b = one(send_addr(1), recv_addr(1))
    assert lib.rc_rank_all_reduce(1, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_OK
    t.join(timeout=30)
    assert first["rc"] == rr.RC_OK
    assert lib.rc_rank_finish(0) == rr.RC_OK


def test_single_rank_does_not_wait(lib):
    assert lib.rc_rank_register(0, 1, ctypes.byref(cfg())) == rr.RC_OK
    b = one(send_addr(0), recv_addr(0))
    assert lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_OK
    assert lib.rc_rank_finish(0) == rr.RC_OK


def test_finish_releases_ranks_waiting_for_it(lib):
    # rank 2 finishes instead of joining the all_reduce the others wait in
    R = 3
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK

    def body(r):
        if r == 2:
            time.sleep(0.3)
            return lib.rc_rank_finish(2)
        b = one(send_addr(r), recv_addr(r))
        rc = lib.rc_rank_all_reduce(r, ctypes.cast(b, ctypes.c_void_p), None)
        return rc, lib.rc_last_error().decode()

    res = run_ranks(R, body)
    assert res[2] == rr.RC_OK
    for r in range(2):
        assert res[r][0] == rr.RC_ERR_NOT_REGISTERED
        assert "rank 2" in res[r][1] and "finished" in res[r][1]
    # later calls on the world are refused at once rather than waiting
    b = one(send_addr(0), recv_addr(0))
    assert lib.rc_rank_all_reduce(0, ctypes.cast(b, ctypes.c_void_p), None) == rr.RC_ERR_NOT_REGISTERED
    assert lib.rc_rank_barrier(1, None) == rr.RC_ERR_NOT_REGISTERED
    # the ranks left can still finish, which closes the session
    assert lib.rc_rank_finish(0) == rr.RC_OK
    assert lib.rc_rank_finish(1) == rr.RC_OK
    assert lib.rc_rank_register(0, 2, ctypes.byref(cfg())) == rr.RC_OK


def test_finish_releases_a_waiting_send_and_refuses_later_ones(lib):
    R = 3
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK

    def body(r):
        if r == 1:
            time.sleep(0.3)
            return lib.rc_rank_finish(1)
        if r == 0:
            b = one(send_addr(0), recv_addr(0))
            return lib.rc_rank_send(0, ctypes.cast(b, ctypes.c_void_p), 1, None)
        return rr.RC_OK

    assert run_ranks(R, body) == [rr.RC_ERR_NOT_REGISTERED, rr.RC_OK, rr.RC_OK]
    b = one(send_addr(2), recv_addr(2))
    assert lib.rc_rank_recv(2, ctypes.cast(b, ctypes.c_void_p), 1, None) == rr.RC_ERR_NOT_REGISTERED
    assert "has finished" in lib.rc_last_error().decode()
    # pairs between ranks still registered are unaffected
    res = run_ranks(R, lambda r: (
        lib.rc_rank_send(0, ctypes.cast(one(send_addr(0), recv_addr(0)), ctypes.c_void_p), 2, None) if r == 0 else
        lib.rc_rank_recv(2, ctypes.cast(one(send_addr(2), recv_addr(2)), ctypes.c_void_p), 0, None) if r == 2 else
        rr.RC_OK))
    assert res == [rr.RC_OK] * R
