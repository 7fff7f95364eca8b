"""The Communicator page's copies on the GPU, bit for bit against the CPU
oracle: list-form all_gather, all_to_all_single and send/recv from one call
and from one thread per rank, and barrier ordering between the ranks'
streams."""

import threading

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import assert_bits, host, session

pytestmark = pytest.mark.gpu
DEV = "cuda"


def view_at(n, offset, dtype=torch.float32, fill=None):
    """A tensor of n elements starting `offset` elements into a fresh buffer
    (misaligned for offset % 4 != 0)."""
    base = torch.empty(n + offset + 4, dtype=dtype, device=DEV)
    t = base[offset:offset + n]
    if fill is not None:
        t.copy_(fill)
    return t


def inputs(R, n, dtype, seed, offsets=None):
    xs = si.torch_rank_inputs(R, n, "i32" if dtype == torch.int32 else "f32", "normal", seed, device=DEV)
    if offsets:
        xs = [view_at(n, offsets[r % len(offsets)], dtype, x) for r, x in enumerate(xs)]
    return xs


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("m", [0, 1, 257, 65_537])
def test_all_gather_list(R, m):
    xs = inputs(R, m, torch.float32, 200 + R, offsets=[0, 1, 2, 3] if m > 1 else None)
    with session(R, device=0):
        out = rr.all_gather_list(xs)
        torch.cuda.synchronize()
    want = oracle.all_gather_list([host(x) for x in xs])
    for r in range(R):
        for k in range(R):
            assert_bits(host(out[r][k]), want[r][k], f"R={R} m={m} rank {r} shard {k}")


@pytest.mark.parametrize("R", [2, 8, 16])
def test_copy_batches_whole_tiles(R):
    """Shards of whole 512-element tiles on aligned buffers: the copy batches
    passed by value run the whole-tile copy kernel (the all_to_all of 16 ranks
    has too many pointers for the kernel arguments and keeps the table path)."""
    m = 65_536
    xs = inputs(R, m, torch.float32, 230 + R)
    ys = inputs(R, R * m, torch.int32, 240 + R)
    with session(R, device=0):
        gl = rr.all_gather_list(xs)
        a2a = rr.all_to_all_single(ys)
        torch.cuda.synchronize()
    want = oracle.all_gather_list([host(x) for x in xs])
    want_a2a = oracle.all_to_all_single([host(y) for y in ys])
    for r in range(R):
        assert_bits(host(a2a[r]), want_a2a[r], f"all_to_all R={R} rank {r}")
        for k in range(R):
            assert_bits(host(gl[r][k]), want[r][k], f"all_gather_list R={R} rank {r} shard {k}")


def test_copy_batches_keep_bits_while_tuned():
    """Copy batches large enough for the occupancy tuner (the list all_gather
    of 8 shards of 8 MiB, all_to_all_single of 8 x 32 MiB) through and past
    its calibration launches: every call equals the oracle bit for bit."""
    R, M = 8, 2 * 2**20
    xs = inputs(R, M, torch.float32, 250)
    ys = inputs(R, 4 * M, torch.int32, 251)
    want = oracle.all_gather_list([host(x) for x in xs])
    want_a2a = oracle.all_to_all_single([host(y) for y in ys])
    with session(R, device=0):
        for call in range(10):
            gl = rr.all_gather_list(xs)
            a2a = rr.all_to_all_single(ys)
            torch.cuda.synchronize()
            r = call % R
            assert_bits(host(a2a[r]), want_a2a[r], f"call {call} all_to_all rank {r}")
            for k in (0, R - 1):
                assert_bits(host(gl[r][k]), want[r][k], f"call {call} all_gather_list rank {r} shard {k}")


def test_all_gather_list_own_slot_in_place_i32():
    R = 4
    m = 10_001
    xs = inputs(R, m, torch.int32, 211)
    keep = [host(x).copy() for x in xs]
    out = [[xs[k] if k == r else torch.empty_like(xs[k]) for k in range(R)] for r in range(R)]
    with session(R, device=0):
        rr.all_gather_list(xs, out=out)
        torch.cuda.synchronize()
    for r in range(R):
        for k in range(R):
            assert_bits(host(out[r][k]), keep[k], f"rank {r} shard {k}")


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("m", [0, 1, 3, 257, 40_000])
def test_all_to_all_single(R, m):
    n = R * m
    xs = inputs(R, n, torch.float32, 300 + R, offsets=[0, 3, 1] if n > 1 else None)
    with session(R, device=0):
        out = rr.all_to_all_single(xs)
        torch.cuda.synchronize()
    want = oracle.all_to_all_single([host(x) for x in xs])
    for r in range(R):
        assert_bits(host(out[r]), want[r], f"R={R} m={m} rank {r}")


def test_all_to_all_single_2d_i32():
    R = 4
    xs = [si.torch_tensor_for(7, 0, R, r, (8, 1000), dtype="i32", device=DEV) for r in range(R)]
    with session(R, device=0):
        out = rr.all_to_all_single(xs)
        torch.cuda.synchronize()
    want = oracle.all_to_all_single([host(x) for x in xs])
    for r in range(R):
        assert out[r].shape == (8, 1000)
        assert_bits(host(out[r]), want[r], f"rank {r}")


@pytest.mark.parametrize("n", [0, 1, 7, 1_000_003])
def test_send_recv_whole_call(n):
    R = 4
    x = inputs(1, n, torch.float32, 400 + n)[0]
    with session(R, device=0):
        y = rr.send_recv(x, 3, 1)
        z = rr.send_recv(x, 0, 2, out=view_at(n, 1))
        rr.barrier()
        torch.cuda.synchronize()
    assert_bits(host(y), oracle.send_recv(host(x)), "send_recv")
    assert_bits(host(z), oracle.send_recv(host(x)), "send_recv into a misaligned view")


# ---------------------------------------------------------------- per rank

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
        t.join(timeout=120)
    assert not errs, errs
    assert all(not t.is_alive() for t in ts)
    return out


def slow_copy(src):
    """An exact copy built through a chain of kernels, still running when the
    next call is issued."""
    x = src.clone()
    for _ in range(6):
        x = (x * 2.0 - x) / 1.0
    return x


@pytest.mark.parametrize("n_streams", [1, 4])
def test_rank_threads_copies(n_streams):
    R = 4
    m = 300_001
    xs = inputs(R, R * m, torch.float32, 500)
    shards = inputs(R, m, torch.float32, 501)
    torch.cuda.synchronize()
    hx = [host(x) for x in xs]
    hs = [host(s) for s in shards]
    pool = [torch.cuda.Stream() for _ in range(n_streams)]
    for r in range(R):
        rr.rank_register(r, R, device=0)

    def body(r):
        s = pool[r % n_streams]
        res = {}
        with torch.cuda.stream(s):
            x = slow_copy(xs[r])
            res["a2a"] = rr.rank_all_to_all_single(r, x, stream=s).clone()
            x.mul_(0)
            sh = slow_copy(shards[r])
            res["list"] = [o.clone() for o in rr.rank_all_gather_list(r, sh, R, stream=s)]
            sh.mul_(0)
            # ring exchange: even ranks send first, odd ranks receive first
            nxt, prv = (r + 1) % R, (r - 1) % R
            mine = slow_copy(shards[r])
            got = torch.empty_like(mine)
            if r % 2 == 0:
                rr.rank_send(r, mine, nxt, stream=s)
                rr.rank_recv(r, got, prv, stream=s)
            else:
                rr.rank_recv(r, got, prv, stream=s)
                rr.rank_send(r, mine, nxt, stream=s)
            res["p2p"] = got.clone()
            mine.mul_(0)
        return res

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        want_a2a = oracle.all_to_all_single(hx)
        want_list = oracle.all_gather_list(hs)
        for r in range(R):
            assert_bits(host(got[r]["a2a"]), want_a2a[r], f"a2a rank {r}")
            for k in range(R):
                assert_bits(host(got[r]["list"][k]), want_list[r][k], f"list rank {r} shard {k}")
            assert_bits(host(got[r]["p2p"]), oracle.send_recv(hs[(r - 1) % R]), f"p2p rank {r}")
    finally:
        for r in range(R):
            rr.rank_finish(r)


def test_rank_barrier_orders_streams():
    """Each rank fills its slot of a shared buffer on its own stream, then
    calls the barrier; afterwards every rank copies the whole buffer on its
    stream.  Only the barrier's stream join orders those reads after the
    other ranks' fills."""
    R = 4
    n = 2_000_000
    src = inputs(R, n, torch.float32, 600)
    shared = torch.zeros(R, n, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    pool = [torch.cuda.Stream() for _ in range(R)]
    for r in range(R):
        rr.rank_register(r, R, device=0)

    def body(r):
        with torch.cuda.stream(pool[r]):
            shared[r].copy_(slow_copy(src[r]))
            rr.rank_barrier(r, stream=pool[r])
            return shared.clone()

    try:
        seen = run_ranks(R, body)
        torch.cuda.synchronize()
        want = np.stack([host(x) for x in src])
        for r in range(R):
            assert_bits(host(seen[r]), want, f"rank {r} after the barrier")
    finally:
        for r in range(R):
            rr.rank_finish(r)


# ---------------------------------------------------------------- destinations off their bursts

PAD = 32


def padded(n, offset, dtype=torch.float32):
    """(base, view): n elements `offset` into a buffer of sentinels."""
    from gpu_util import SENTINEL
    base = torch.full((n + PAD,), SENTINEL, dtype=torch.int32, device=DEV)
    base = base.view(dtype) if dtype == torch.float32 else base
    return base, base[offset:offset + n]


def pads_intact(base, offset, n, what):
    from gpu_util import SENTINEL
    hb = host(base).view(np.uint32)
    assert np.all(hb[:offset] == SENTINEL) and np.all(hb[offset + n:] == SENTINEL), \
        f"{what}: written outside its destination (offset {offset})"


@pytest.mark.parametrize("R", [2, 3, 4, 8, 16])
def test_copies_to_destinations_off_bursts(R):
    """Whole-tile copies whose destinations start 1-15 elements past a 64-byte
    boundary (sources and rank 0's destination aligned, so the jobs stay whole
    tiles): the shifted copy kernels write those destinations over
    burst-aligned ranges.  broadcast (also from a sender whose own buffer is
    its output), all_gather, the list all_gather (odd ranks' destinations
    off), and the ring all-reduce's copy phase; sentinels around every
    destination; bits against the oracle."""
    M = 8192  # whole tiles of the copy kernels (512 elements), several per job
    N = R * M
    offs = [0] + [1 + (5 * r) % 15 for r in range(1, R)]
    xs = inputs(R, N, torch.float32, 900 + R)
    hx = [host(x).copy() for x in xs]
    with session(R):
        for root in (0, R - 1):
            bufs = [padded(N, o) for o in offs]
            sends = [xs[r] if r == root else None for r in range(R)]
            rr.broadcast(sends, out=[v if r != root else None for r, (_, v) in enumerate(bufs)])
            torch.cuda.synchronize()
            for r, (b, v) in enumerate(bufs):
                if r == root:
                    continue
                assert_bits(host(v), hx[root], f"broadcast R={R} from {root} rank {r}")
                pads_intact(b, offs[r], N, f"broadcast rank {r}")
        # the sender's own output is its input: only the receivers are written
        root = R - 1
        sb, sv = padded(N, 0)
        sv.copy_(xs[root])
        bufs = [padded(N, o) for o in offs]
        outs = [v for _, v in bufs]
        outs[root] = sv
        rr.broadcast([sv if r == root else None for r in range(R)], out=outs)
        torch.cuda.synchronize()
        for r in range(R):
            assert_bits(host(outs[r]), hx[root], f"broadcast in place R={R} rank {r}")
        shards = [x[:M].clone() for x in xs]
        hs = [host(s) for s in shards]
        bufs = [padded(N, o) for o in offs]
        rr.all_gather(shards, out=[v for _, v in bufs])
        torch.cuda.synchronize()
        want = oracle.all_gather(hs)
        for r, (b, v) in enumerate(bufs):
            assert_bits(host(v), want[r], f"all_gather R={R} rank {r}")
            pads_intact(b, offs[r], N, f"all_gather rank {r}")
        lst_bufs = [[padded(M, 0 if r % 2 == 0 else 1 + (3 * r + 7 * k) % 15) for k in range(R)] for r in range(R)]
        rr.all_gather_list(shards, out=[[v for _, v in row] for row in lst_bufs])
        torch.cuda.synchronize()
        for r in range(R):
            for k in range(R):
                b, v = lst_bufs[r][k]
                assert_bits(host(v), hs[k], f"all_gather_list R={R} rank {r} shard {k}")
                pads_intact(b, 0 if r % 2 == 0 else 1 + (3 * r + 7 * k) % 15, M, f"all_gather_list {r}/{k}")
    with session(R, algo="ring"):
        bufs = [padded(N, o) for o in offs]
        rr.all_reduce(xs, "sum", out=[v for _, v in bufs])
        torch.cuda.synchronize()
        want = oracle.all_reduce_closed_form(hx, "sum")
        for r, (b, v) in enumerate(bufs):
            assert_bits(host(v), want, f"ring all_reduce R={R} rank {r}")
            pads_intact(b, offs[r], N, f"ring all_reduce rank {r}")
    for r in range(R):
        assert_bits(host(xs[r]), hx[r], f"input of rank {r} changed")
