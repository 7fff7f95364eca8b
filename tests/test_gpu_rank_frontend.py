"""The per-rank front end on the GPU: one host thread and one stream per
logical rank.  Each rank produces its input on its own stream right before
its call and consumes the output on that stream right after, with no host
synchronisation in between, so the results are only right if the library
orders the kernels after every rank's producer and every consumer after the
kernels.  Bits are compared with the CPU oracle."""

import random
import threading

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import assert_bits, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


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
    """src, rebuilt through a chain of exact float32 ops (x*2-x = x, x/1 = x),
    so the producer is still running when the rank's call is issued."""
    x = src.clone()
    for _ in range(6):
        x = (x * 2.0 - x) / 1.0
    return x


def test_rank_threads_through_tuner_calibration():
    """Eight rank threads on eight streams, calls large enough for the
    occupancy tuner (256 MiB moved), ten in a row: the timed launches sit on
    the launching rank's stream between the joins, and every call's result
    is the oracle's, consumed on each rank's own stream."""
    R, N = 8, 4 * 2**20
    srcs = si.torch_rank_inputs(R, N, "f32", "normal", 90, device=DEV)
    torch.cuda.synchronize()
    want = oracle.all_reduce([host(x) for x in srcs], "sum")
    streams = [torch.cuda.Stream() for _ in range(R)]
    for r in range(R):
        rr.rank_register(r, R)

    def body(r):
        outs = []
        with torch.cuda.stream(streams[r]):
            for _ in range(10):
                x = slow_copy(srcs[r])
                out = rr.rank_all_reduce(r, x, "sum", stream=streams[r])
                outs.append(out.clone())  # consumer on the rank's stream
        return outs

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        for r in range(R):
            for k, o in enumerate(got[r]):
                assert_bits(host(o), want[r], f"call {k} rank {r}")
    finally:
        for r in range(R):
            rr.rank_finish(r)


@pytest.mark.parametrize("R,n_streams", [(2, 2), (4, 4), (8, 8), (8, 1), (6, 3)])
def test_rank_threads_all_reduce(R, n_streams):
    """Rank r on stream r mod n_streams: own streams, one shared stream (no
    events), and pairs of ranks sharing a stream."""
    N = 4_000_037
    srcs = si.torch_rank_inputs(R, N, "f32", "normal", 70 + R, device=DEV)
    torch.cuda.synchronize()
    hx = [host(x) for x in srcs]
    pool = [torch.cuda.Stream() for _ in range(n_streams)]
    streams = [pool[r % n_streams] for r in range(R)]
    for r in range(R):
        rr.rank_register(r, R)

    def body(r):
        got = {}
        with torch.cuda.stream(streams[r]):
            for op in ("sum", "mean", "max"):
                x = slow_copy(srcs[r])
                out = rr.rank_all_reduce(r, x, op, stream=streams[r])
                got[op] = out.clone()  # consumer on the rank's stream
                x.mul_(0)              # overwrite the input right after the call
        return got

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        for op in ("sum", "mean", "max"):
            want = oracle.all_reduce_closed_form(hx, op)
            for r in range(R):
                assert_bits(host(got[r][op]), want, f"R={R} {op} rank {r}")
    finally:
        for r in range(R):
            rr.rank_finish(r)


def test_rank_threads_every_collective():
    R = 4
    M = 250_007
    N = R * M
    srcs = si.torch_rank_inputs(R, N, "i32", "int", 81, device=DEV)
    torch.cuda.synchronize()
    hx = [host(x) for x in srcs]
    streams = [torch.cuda.Stream() for _ in range(R)]
    for r in range(R):
        rr.rank_register(r, R)

    def body(r):
        s = streams[r]
        res = {}
        with torch.cuda.stream(s):
            x = srcs[r].clone()
            out = rr.rank_reduce(r, x, 2, "sum", stream=s)
            res["reduce"] = out.clone() if out is not None else None
            b_out = torch.empty_like(x) if r != 1 else None
            res["broadcast"] = rr.rank_broadcast(r, x if r == 1 else None, out=b_out, stream=s)
            if r != 1:
                res["broadcast"] = res["broadcast"].clone()
            res["rs"] = rr.rank_reduce_scatter(r, x, R, "max", stream=s).clone()
            shard = (x[:M] + 0).contiguous()
            res["ag"] = rr.rank_all_gather(r, shard, R, stream=s).clone()
        return res

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        assert_bits(host(got[2]["reduce"]), oracle.reduce(hx, 2, "sum")[2], "reduce root 2")
        for r in (0, 2, 3):
            assert_bits(host(got[r]["broadcast"]), hx[1], f"broadcast rank {r}")
        want_rs = oracle.reduce_scatter(hx, "max")
        want_ag = np.concatenate([h[:M] for h in hx])
        for r in range(R):
            assert_bits(host(got[r]["rs"]), want_rs[r], f"reduce_scatter rank {r}")
            assert_bits(host(got[r]["ag"]), want_ag, f"all_gather rank {r}")
    finally:
        for r in range(R):
            rr.rank_finish(r)


def test_rank_mismatch_on_gpu_launches_nothing():
    R = 2
    xs = si.torch_rank_inputs(R, 1000, "f32", "normal", 5, device=DEV)
    outs = [torch.full_like(x, 7.0) for x in xs]
    for r in range(R):
        rr.rank_register(r, R)

    def body(r):
        op = "sum" if r == 0 else "max"
        try:
            rr.rank_all_reduce(r, xs[r], op, out=outs[r])
        except rr.CollectiveError as e:
            return e.code
        return rr.RC_OK

    try:
        assert run_ranks(R, body) == [rr.RC_ERR_OP_MISMATCH] * R
        torch.cuda.synchronize()
        for o in outs:
            assert torch.all(o == 7.0).item(), "an output was written despite the error"
    finally:
        for r in range(R):
            rr.rank_finish(r)


def test_split_groups_reduce_in_their_own_rank_order():
    """Eight rank threads split into two communicators (world ranks 0,2,4,6
    and 7,5,3,1, in those orders); each group all-reduces its members'
    tensors concurrently with the other, folding in the group's own ring
    order, and reduces to its rank 1."""
    R = 8
    N = 1_000_003
    xs = si.torch_rank_inputs(R, N, "f32", "normal", 90, device=DEV)
    torch.cuda.synchronize()
    hx = [host(x) for x in xs]
    groups = [[0, 2, 4, 6], [7, 5, 3, 1]]
    streams = [torch.cuda.Stream() for _ in range(R)]
    for r in range(R):
        rr.rank_register(r, R, device=0)

    def body(r):
        g = 0 if r % 2 == 0 else 1
        eps = [rr.rank_split(r, groups[i] if i == g else []) for i in range(2)]
        ep = eps[g]
        assert eps[1 - g] is None
        s = streams[r]
        with torch.cuda.stream(s):
            out = rr.rank_all_reduce(ep, xs[r], "sum", stream=s).clone()
            red = rr.rank_reduce(ep, xs[r], 1, "mean", stream=s)
            red = red.clone() if red is not None else None
        rr.rank_finish(ep)
        return g, out, red

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        for g, members in enumerate(groups):
            gx = [hx[w] for w in members]
            want = oracle.all_reduce_closed_form(gx, "sum")
            want_mean = oracle.reduce(gx, 1, "mean")[1]
            for i, w in enumerate(members):
                assert got[w][0] == g
                assert_bits(host(got[w][1]), want, f"group {g} world rank {w}")
                if i == 1:
                    assert_bits(host(got[w][2]), want_mean, f"group {g} reduce at its rank 1")
                else:
                    assert got[w][2] is None
    finally:
        for r in range(R):
            rr.rank_finish(r)


def _plan_sequence(rng, R, count):
    """`count` collectives of random kinds, sizes, types and roots, the same
    for every rank (a send/recv pair involves two ranks only)."""
    kinds = ["all_reduce", "reduce", "broadcast", "reduce_scatter", "all_gather", "all_gather_list",
             "all_to_all_single", "barrier", "params", "send_recv"]
    plan = []
    for _ in range(count):
        kind = rng.choice(kinds)
        dtype = rng.choice(["f32", "i32"])
        op = rng.choice(["sum", "max"] if dtype == "i32" else ["sum", "mean", "max"])
        n = rng.choice([1, 257, 4099, R * 2048, rng.randint(1, 150_000)])
        if kind in ("reduce_scatter", "all_to_all_single"):
            n = max(R, n - n % R)
        if kind == "params":
            op = "sum" if dtype == "i32" else rng.choice(["sum", "mean"])
        pair = rng.sample(range(R), 2)
        plan.append({"kind": kind, "dtype": dtype, "op": op, "n": n, "root": rng.randrange(R),
                     "pair": pair, "acc": rng.random() < 0.5})
    return plan


@pytest.mark.parametrize("seed", [1, 2, 4, 5, 6, 9, 21, 24, 25, 30])
def test_rank_threads_random_sequences(seed):
    """A seeded sequence of 24 collectives of every kind, issued by R rank
    threads in the same order, with the ranks spread over 1 to R streams
    (seeds chosen for 2 to 8 ranks on one stream, on some shared streams and
    on a stream each).
    Each rank produces its input on its stream right before each call,
    consumes the output right after, and then overwrites its input: every
    consumed output equals the oracle's, so every call ran after every
    rank's producer and before every rank's later work."""
    rng = random.Random(7_000 + seed)
    R = rng.choice([2, 3, 4, 5, 8])
    S = rng.choice(sorted({1, 2, R}))
    plan = _plan_sequence(rng, R, 24)
    gen_ = torch.Generator(device=DEV).manual_seed(seed)
    srcs, accs = [], []
    for p in plan:
        if p["dtype"] == "i32":
            draw = [torch.randint(-2 ** 20, 2 ** 20 + 1, (p["n"],), dtype=torch.int32, device=DEV, generator=gen_)
                    for _ in range(R)]
            dacc = [torch.randint(-2 ** 20, 2 ** 20 + 1, (p["n"],), dtype=torch.int32, device=DEV, generator=gen_)
                    for _ in range(R)]
        else:
            draw = [torch.randn(p["n"], device=DEV, generator=gen_) for _ in range(R)]
            dacc = [torch.randn(p["n"], device=DEV, generator=gen_) for _ in range(R)]
        srcs.append(draw)
        accs.append(dacc)
    torch.cuda.synchronize()
    hx = [[host(x) for x in xs] for xs in srcs]
    ha = [[host(a) for a in xs] for xs in accs]
    pool = [torch.cuda.Stream() for _ in range(S)]
    for r in range(R):
        rr.rank_register(r, R)

    def body(r):
        s = pool[r % S]
        got = []
        with torch.cuda.stream(s):
            for i, p in enumerate(plan):
                kind, op, n = p["kind"], p["op"], p["n"]
                x = slow_copy(srcs[i][r]) if p["dtype"] == "f32" else srcs[i][r].clone()  # producer
                res = None
                if kind == "all_reduce":
                    res = rr.rank_all_reduce(r, x, op, stream=s)
                elif kind == "reduce":
                    res = rr.rank_reduce(r, x, p["root"], op, stream=s)
                elif kind == "broadcast":
                    src = p["root"]
                    res = rr.rank_broadcast(r, x if r == src else None,
                                            out=None if r == src else torch.empty_like(x), stream=s)
                elif kind == "reduce_scatter":
                    res = rr.rank_reduce_scatter(r, x, R, op, stream=s)
                elif kind == "all_gather":
                    res = rr.rank_all_gather(r, x, R, stream=s)
                elif kind == "all_gather_list":
                    res = torch.cat(rr.rank_all_gather_list(r, x, R, stream=s))
                elif kind == "all_to_all_single":
                    res = rr.rank_all_to_all_single(r, x, stream=s)
                elif kind == "barrier":
                    rr.rank_barrier(r, stream=s)
                elif kind == "params":
                    acc = {5: accs[i][r].clone()} if p["acc"] else None
                    res = rr.rank_all_reduce_params(r, {5: x}, op, stream=s, acc=acc)[5]
                else:
                    a, b = p["pair"]
                    if r == a:
                        rr.rank_send(r, x, b, stream=s)
                    elif r == b:
                        res = rr.rank_recv(r, torch.empty_like(x), a, stream=s)
                got.append(res.clone() if res is not None else None)  # consumer
                x.mul_(0)  # the rank's next use of its input buffer
        return got

    try:
        got = run_ranks(R, body)
        torch.cuda.synchronize()
        for i, p in enumerate(plan):
            kind, op, xs = p["kind"], p["op"], hx[i]
            what = f"seed {seed} R={R} S={S} call {i}: {kind} {p['dtype']} {op} n={p['n']}"
            if kind == "all_reduce":
                want = oracle.all_reduce(xs, op)
            elif kind == "reduce":
                want = oracle.reduce(xs, p["root"], op)
            elif kind == "broadcast":
                want = oracle.broadcast([x if r == p["root"] else None for r, x in enumerate(xs)])
                want[p["root"]] = None  # the sender asked for no output
            elif kind == "reduce_scatter":
                want = oracle.reduce_scatter(xs, op)
            elif kind == "all_gather":
                want = oracle.all_gather(xs)
            elif kind == "all_gather_list":
                want = [np.concatenate(w) for w in oracle.all_gather_list(xs)]
            elif kind == "all_to_all_single":
                want = oracle.all_to_all_single(xs)
            elif kind == "barrier":
                want = [None] * R
            elif kind == "params":
                acc = [{5: a} for a in ha[i]] if p["acc"] else None
                w = oracle.all_reduce_params([{5: x} for x in xs], op, acc=acc)
                want = [m[5] for m in w]
            else:
                a, b = p["pair"]
                want = [oracle.send_recv(xs[a]) if r == b else None for r in range(R)]
            for r in range(R):
                if want[r] is None:
                    assert got[r][i] is None, f"{what}: rank {r} got an output"
                else:
                    assert_bits(host(got[r][i]), want[r], f"{what}: rank {r}")
    finally:
        for r in range(R):
            rr.rank_finish(r)
