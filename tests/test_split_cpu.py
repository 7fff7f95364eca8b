"""Communicator splits on the CPU (validate-only sessions, fake addresses):
split_from and split_all of the per-rank front end, collectives on the new
communicators with ranks counted inside them, nesting, errors, and finish."""

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


def split(lib, ep, members):
    arr = (ctypes.c_int * max(len(members), 1))(*members)
    out = ctypes.c_int(-7)
    rc = lib.rc_rank_split(ep, len(members), arr, ctypes.byref(out))
    return rc, out.value


def ar(lib, ep, world_rank, n=1024):
    b = rr.make_bufs([0x100000000 + world_rank * 64 * MiB], [0x800000000 + world_rank * 64 * MiB], (n,))
    return lib.rc_rank_all_reduce(ep, ctypes.cast(b, ctypes.c_void_p), None)


def test_split_from_even_odd_and_collectives(lib):
    R = 6

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        evens, odds = [0, 2, 4], [5, 3, 1]
        rc1, e_ep = split(lib, r, evens if r % 2 == 0 else [])
        rc2, o_ep = split(lib, r, odds if r % 2 == 1 else [])
        res = [rc1, rc2, e_ep, o_ep]
        mine = e_ep if r % 2 == 0 else o_ep
        # collectives inside the group: three members, ranks counted within it
        for _ in range(5):
            res.append(ar(lib, mine, r))
        res.append(lib.rc_rank_barrier(mine, None))
        # the world still works
        res.append(ar(lib, r, r))
        res.append(lib.rc_rank_finish(mine))
        res.append(ar(lib, mine, r))        # finished endpoint
        res.append(lib.rc_rank_finish(r))
        return res

    out = run_ranks(R, body)
    for r, res in enumerate(out):
        assert res[:2] == [rr.RC_OK, rr.RC_OK]
        if r % 2 == 0:
            assert res[2] == 1 * rr.RC_MAX_RANKS + [0, 2, 4].index(r) and res[3] == -1
        else:
            assert res[2] == -1 and res[3] == 2 * rr.RC_MAX_RANKS + [5, 3, 1].index(r)
        assert res[4:11] == [rr.RC_OK] * 7
        assert res[11] == rr.RC_OK
        assert res[12] == rr.RC_ERR_NOT_REGISTERED
        assert res[13] == rr.RC_OK


def test_split_all_and_nesting(lib):
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        rc, same = split(lib, r, list(range(R)))           # split_all
        assert rc == rr.RC_OK and same == 1 * rr.RC_MAX_RANKS + r
        # a pair out of the split-off communicator: its ranks 3 and 0, in that order
        rc, pair = split(lib, same, [3, 0] if r in (0, 3) else [])
        assert rc == rr.RC_OK
        res = [pair]
        if pair is not None and pair >= 0:
            res.append(ar(lib, pair, r))
            # send/recv inside the pair, peers counted in the pair
            b = rr.make_bufs([0x100000000 + r * 64 * MiB], [0x800000000 + r * 64 * MiB], (64,))
            if pair % rr.RC_MAX_RANKS == 0:
                res.append(lib.rc_rank_send(pair, ctypes.cast(b, ctypes.c_void_p), 1, None))
            else:
                res.append(lib.rc_rank_recv(pair, ctypes.cast(b, ctypes.c_void_p), 0, None))
        res.append(ar(lib, same, r))
        return res

    out = run_ranks(R, body)
    for r in (0, 3):
        assert out[r][0] == 2 * rr.RC_MAX_RANKS + [3, 0].index(r)
        assert out[r][1:] == [rr.RC_OK] * 3
    for r in (1, 2):
        assert out[r] == [-1, rr.RC_OK]


def test_split_errors_reach_every_rank(lib):
    R = 4

    def body(r):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
        res = []
        res.append(split(lib, r, [0, 1] if r != 1 else [1, 0]))    # different lists
        res.append(split(lib, r, [0, 1] if r == 0 else []))         # rank 1 listed, passed none
        res.append(split(lib, r, [0, 0] if r == 0 else []))         # duplicate
        res.append(split(lib, r, [0, 4] if r == 0 else []))         # out of range
        res.append(lib.rc_rank_split(r, 2, None, None) if r == 2 else split(lib, r, [])[0])
        res.append(split(lib, r, []))                               # nobody named: no communicator
        res.append(ar(lib, r, r))                                   # the world is fine
        return res

    for res in run_ranks(R, body):
        for item in res[:4]:
            assert item == (rr.RC_ERR_INVALID_ARGUMENT, -1)
        assert res[4] == rr.RC_ERR_INVALID_ARGUMENT
        assert res[5] == (rr.RC_OK, -1)
        assert res[6] == rr.RC_OK


def test_unknown_endpoints(lib):
    R = 2
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
    assert ar(lib, 5 * rr.RC_MAX_RANKS, 0) == rr.RC_ERR_NOT_REGISTERED
    assert ar(lib, R, 0) == rr.RC_ERR_INVALID_ARGUMENT
    assert lib.rc_rank_finish(3 * rr.RC_MAX_RANKS + 1) == rr.RC_ERR_NOT_REGISTERED


def test_leaving_a_split_communicator_releases_its_members(lib):
    # world of 4; {0, 1, 2} split off.  Member 2 leaves the split communicator
    # while 0 and 1 wait in it; then world rank 3 finishes, which releases
    # world rank 0's wait on the world.
    R = 4
    for r in range(R):
        assert lib.rc_rank_register(r, R, ctypes.byref(cfg())) == rr.RC_OK
    eps = run_ranks(R, lambda r: split(lib, r, [0, 1, 2] if r < 3 else []))
    assert [rc for rc, _ in eps] == [rr.RC_OK] * R
    sub = [ep for _, ep in eps]
    assert sub[3] == -1

    def body(r):
        if r == 2:
            time.sleep(0.3)
            return lib.rc_rank_finish(sub[2])
        if r == 3:
            return rr.RC_OK
        return ar(lib, sub[r], r)

    assert run_ranks(R, body) == [rr.RC_ERR_NOT_REGISTERED, rr.RC_ERR_NOT_REGISTERED, rr.RC_OK, rr.RC_OK]
    # the split communicator refuses further calls; the world still works
    assert ar(lib, sub[0], 0) == rr.RC_ERR_NOT_REGISTERED
    assert run_ranks(R, lambda r: ar(lib, r, r)) == [rr.RC_OK] * R

    def body2(r):
        if r == 3:
            time.sleep(0.3)
            return lib.rc_rank_finish(3)
        if r == 0:
            return ar(lib, 0, 0)
        return rr.RC_OK

    assert run_ranks(R, body2) == [rr.RC_ERR_NOT_REGISTERED, rr.RC_OK, rr.RC_OK, rr.RC_OK]
    for ep in (sub[0], sub[1]):
        assert lib.rc_rank_finish(ep) == rr.RC_OK
    for r in range(3):
        assert lib.rc_rank_finish(r) == rr.RC_OK
