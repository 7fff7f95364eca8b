"""The Communicator page's other methods on the CPU (validate-only sessions,
fake addresses): list-form all_gather, all_to_all_single, send/recv and
barrier, from the whole-call and the per-rank entry points, with every
argument error."""

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


def send_addr(r):
    return 0x100000000 + r * 64 * MiB


def recv_addr(r, k=0):
    return 0x800000000 + r * 64 * MiB + k * MiB


def err(lib):
    return lib.rc_last_error().decode()


def gather_list(lib, R, m=1000, edit=None, recv_edit=None):
    bufs = rr.make_bufs([send_addr(r) for r in range(R)], [None] * R, (m,))
    recvs = [recv_addr(r, k) for r in range(R) for k in range(R)]
    if edit:
        edit(bufs)
    if recv_edit:
        recv_edit(recvs)
    arr = (ctypes.c_void_p * (R * R))(*recvs)
    return lib.rc_all_gather_list(ctypes.cast(bufs, ctypes.c_void_p), arr, None)


def test_all_gather_list_checks(lib):
    R = 4
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    assert gather_list(lib, R) == rr.RC_OK
    assert gather_list(lib, R, m=0) == rr.RC_OK

    def own_in_place(recvs):
        for r in range(R):
            recvs[r * R + r] = send_addr(r)
    assert gather_list(lib, R, recv_edit=own_in_place) == rr.RC_OK

    def other_in_place(recvs):
        recvs[0 * R + 1] = send_addr(1)
    assert gather_list(lib, R, recv_edit=other_in_place) == rr.RC_ERR_INVALID_ARGUMENT

    def clash(recvs):
        recvs[5] = recvs[6]
    assert gather_list(lib, R, recv_edit=clash) == rr.RC_ERR_INVALID_ARGUMENT
    assert "overlaps" in err(lib)

    def null(recvs):
        recvs[7] = None
    assert gather_list(lib, R, recv_edit=null) == rr.RC_ERR_INVALID_ARGUMENT
    assert "NULL" in err(lib)

    def misaligned(recvs):
        recvs[3] += 2
    assert gather_list(lib, R, recv_edit=misaligned) == rr.RC_ERR_INVALID_ARGUMENT

    def shape(bufs):
        bufs[2].dims[0] = 999
    assert gather_list(lib, R, edit=shape) == rr.RC_ERR_SHAPE_MISMATCH
    bufs = rr.make_bufs([send_addr(r) for r in range(R)], [None] * R, (8,))
    assert lib.rc_all_gather_list(ctypes.cast(bufs, ctypes.c_void_p), None, None) == rr.RC_ERR_INVALID_ARGUMENT


def a2a(lib, R, n, edit=None):
    bufs = rr.make_bufs([send_addr(r) for r in range(R)], [recv_addr(r) for r in range(R)], (n,))
    if edit:
        edit(bufs)
    return lib.rc_all_to_all_single(ctypes.cast(bufs, ctypes.c_void_p), None)


def test_all_to_all_checks(lib):
    R = 4
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    assert a2a(lib, R, 4096) == rr.RC_OK
    assert a2a(lib, R, 0) == rr.RC_OK
    assert a2a(lib, R, 4097) == rr.RC_ERR_SHAPE_MISMATCH

    def in_place(bufs):
        bufs[1].recv = bufs[1].send
    assert a2a(lib, R, 4096, in_place) == rr.RC_ERR_INVALID_ARGUMENT

    def dtype(bufs):
        bufs[3].dtype = rr.RC_I32
    assert a2a(lib, R, 4096, dtype) == rr.RC_ERR_DTYPE_MISMATCH

    def null_recv(bufs):
        bufs[0].recv = None
    assert a2a(lib, R, 4096, null_recv) == rr.RC_ERR_INVALID_ARGUMENT


def sr(lib, src, dst, n=100, m=None, dtype=rr.RC_F32, send=None, recv=None):
    bufs = rr.make_bufs([send if send is not None else send_addr(src), None],
                        [None, recv if recv is not None else recv_addr(dst)],
                        [(n,), (m if m is not None else n,)], [rr.RC_F32, dtype])
    return lib.rc_send_recv(src, dst, ctypes.cast(bufs, ctypes.c_void_p), None)


def test_send_recv_and_barrier_checks(lib):
    assert lib.rc_barrier(None) == rr.RC_ERR_NOT_REGISTERED
    R = 3
    assert lib.rc_register(R, ctypes.byref(cfg())) == rr.RC_OK
    assert lib.rc_barrier(None) == rr.RC_OK
    assert sr(lib, 0, 2) == rr.RC_OK
    assert sr(lib, 0, 0) == rr.RC_ERR_INVALID_ARGUMENT
    assert sr(lib, 0, 3) == rr.RC_ERR_INVALID_ARGUMENT
    assert sr(lib, -1, 1) == rr.RC_ERR_INVALID_ARGUMENT
    assert sr(lib, 1, 2, m=101) == rr.RC_ERR_SHAPE_MISMATCH
    assert sr(lib, 1, 2, dtype=rr.RC_I32) == rr.RC_ERR_DTYPE_MISMATCH
    assert sr(lib, 1, 2, recv=send_addr(1)) == rr.RC_OK          # same buffer: nothing moves
    assert sr(lib, 1, 2, recv=send_addr(1) + 8) == rr.RC_ERR_INVALID_ARGUMENT
    assert sr(lib, 1, 2, n=0, send=0, recv=0) == rr.RC_OK
    assert lib.rc_send_recv(0, 1, None, None) == rr.RC_ERR_INVALID_ARGUMENT


# ---------------------------------------------------------------- per rank

def run_ranks(R, body, timeout=60):
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
        t.join(timeout=timeout)
    assert not errs, errs
    assert all(not t.is_alive() for t in ts)
    return out


def one(send, recv, n=1024, dtype=rr.RC_F32):
    return rr.make_bufs([send], [recv], (n,), dtype)


def test_per_rank_copies_and_barrier(lib):
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        res = []
        b = one(send_addr(r), recv_addr(r), n=4096)
        res.append(lib.rc_rank_all_to_all_single(r, ctypes.cast(b, ctypes.c_void_p), None))
        recvs = (ctypes.c_void_p * R)(*[recv_addr(r, k) for k in range(R)])
        b = one(send_addr(r), None, n=1000)
        res.append(lib.rc_rank_all_gather_list(r, ctypes.cast(b, ctypes.c_void_p), recvs, None))
        res.append(lib.rc_rank_barrier(r, None))
        # rank 2 passes no recvs list: every rank hears about it
        res.append(lib.rc_rank_all_gather_list(r, ctypes.cast(b, ctypes.c_void_p), None if r == 2 else recvs,
                                               None))
        # rank 1 calls a barrier where the others call all_to_all
        b = one(send_addr(r), recv_addr(r), n=4096)
        res.append(lib.rc_rank_barrier(r, None) if r == 1 else
                   lib.rc_rank_all_to_all_single(r, ctypes.cast(b, ctypes.c_void_p), None))
        res.append(lib.rc_rank_barrier(r, None))
        res.append(lib.rc_rank_finish(r))
        return res

    for res in run_ranks(R, body):
        assert res == [rr.RC_OK, rr.RC_OK, rr.RC_OK, rr.RC_ERR_INVALID_ARGUMENT, rr.RC_ERR_OP_MISMATCH,
                       rr.RC_OK, rr.RC_OK]


def test_per_rank_send_recv_pairs(lib):
    """Ring exchange (even ranks send first, odd ranks receive first), and
    sends matched per ordered pair whatever the other ranks do."""
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        res = []
        nxt, prv = (r + 1) % R, (r - 1) % R
        s = one(send_addr(r), None)
        d = one(None, recv_addr(r))
        for _ in range(5):
            if r % 2 == 0:
                res.append(lib.rc_rank_send(r, ctypes.cast(s, ctypes.c_void_p), nxt, None))
                res.append(lib.rc_rank_recv(r, ctypes.cast(d, ctypes.c_void_p), prv, None))
            else:
                res.append(lib.rc_rank_recv(r, ctypes.cast(d, ctypes.c_void_p), prv, None))
                res.append(lib.rc_rank_send(r, ctypes.cast(s, ctypes.c_void_p), nxt, None))
        # only ranks 0 and 3 exchange; 1 and 2 go straight to the barrier
        if r == 0:
            res.append(lib.rc_rank_send(r, ctypes.cast(s, ctypes.c_void_p), 3, None))
        if r == 3:
            bad = one(None, recv_addr(r), n=1000)  # shape differs from the sender's
            res.append(lib.rc_rank_recv(r, ctypes.cast(bad, ctypes.c_void_p), 0, None))
        res.append(lib.rc_rank_barrier(r, None))
        res.append(lib.rc_rank_send(r, ctypes.cast(s, ctypes.c_void_p), r, None))   # to itself
        res.append(lib.rc_rank_recv(r, ctypes.cast(d, ctypes.c_void_p), R, None))   # out of range
        res.append(lib.rc_rank_finish(r))
        return res

    out = run_ranks(R, body)
    for r, res in enumerate(out):
        tail = [rr.RC_OK, rr.RC_ERR_INVALID_ARGUMENT, rr.RC_ERR_INVALID_ARGUMENT, rr.RC_OK]
        mid = [rr.RC_ERR_SHAPE_MISMATCH] if r in (0, 3) else []
        assert res == [rr.RC_OK] * 10 + mid + tail, (r, res)


def test_waiting_send_released_by_reset(lib):
    R = 2
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK

    def body(r):
        if r == 1:
            time.sleep(0.3)
            return lib.rc_reset()
        s = one(send_addr(0), None)
        return lib.rc_rank_send(0, ctypes.cast(s, ctypes.c_void_p), 1, None)

    assert run_ranks(R, body) == [rr.RC_ERR_NOT_REGISTERED, rr.RC_OK]
