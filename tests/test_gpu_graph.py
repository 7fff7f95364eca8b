"""Collectives captured into a HIP graph (torch.cuda.CUDAGraph) and replayed:
single collectives and copy batches whose tables travel in the kernel
arguments enqueue nothing but kernels, so every replay recomputes from the
current inputs.  Each replay follows eager work that rewrites the inputs and
a synchronisation, and is checked against the CPU oracle.  The batched
all-reduce, whose tables come from reused host staging, refuses capture
before enqueuing anything."""

import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import assert_bits, host, session

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_replays_follow_the_inputs():
    R = 4
    M = 250_007
    N = R * M
    xs = si.torch_rank_inputs(R, N, "f32", "normal", 700, device=DEV)
    sums = [torch.empty_like(x) for x in xs]
    shards = [torch.empty(M, device=DEV) for _ in range(R)]
    swapped = [torch.empty_like(x) for x in xs]
    with session(R, device=0):
        # warm up outside the capture (first launches load code objects)
        rr.all_reduce(xs, "sum", out=sums)
        rr.reduce_scatter(xs, "max", out=shards)
        rr.all_to_all_single(xs, out=swapped)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rr.all_reduce(xs, "sum", out=sums)
            rr.reduce_scatter(xs, "max", out=shards)
            rr.all_to_all_single(xs, out=swapped)
        for rep in range(4):
            fresh = si.torch_rank_inputs(R, N, "f32", "normal", 710 + rep, device=DEV)
            for x, f in zip(xs, fresh):
                x.copy_(f)  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            hx = [host(x) for x in xs]
            want = oracle.all_reduce_closed_form(hx, "sum")
            want_rs = oracle.reduce_scatter(hx, "max")
            want_a2a = oracle.all_to_all_single(hx)
            for r in range(R):
                assert_bits(host(sums[r]), want, f"replay {rep} all_reduce rank {r}")
                assert_bits(host(shards[r]), want_rs[r], f"replay {rep} reduce_scatter rank {r}")
                assert_bits(host(swapped[r]), want_a2a[r], f"replay {rep} all_to_all rank {r}")


def test_capture_during_occupancy_tuning():
    """An all-reduce large enough for the occupancy tuner, captured while the
    tuner still has timed launches outstanding: the capture makes no event
    calls, replays recompute from the current inputs, and eager calls between
    the replays (which go on tuning) give the same bits."""
    R, N = 8, 4 * 2**20  # 2*R*N*4 = 256 MiB moved: tuned
    xs = si.torch_rank_inputs(R, N, "f32", "normal", 720, device=DEV)
    outs = [torch.empty_like(x) for x in xs]
    eager = [torch.empty_like(x) for x in xs]
    with session(R, device=0):
        rr.all_reduce(xs, "sum", out=outs)  # first timed launches, not read yet
        rr.all_reduce(xs, "sum", out=outs)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rr.all_reduce(xs, "sum", out=outs)
        for rep in range(6):
            fresh = si.torch_rank_inputs(R, N, "f32", "normal", 730 + rep, device=DEV)
            for x, f in zip(xs, fresh):
                x.copy_(f)
            torch.cuda.synchronize()
            g.replay()
            rr.all_reduce(xs, "sum", out=eager)  # eager, tuning goes on
            torch.cuda.synchronize()
            want = oracle.all_reduce([host(x) for x in xs], "sum")
            for r in (0, rep % R, R - 1):
                assert_bits(host(outs[r]), want[r], f"replay {rep} rank {r}")
                assert_bits(host(eager[r]), want[r], f"eager {rep} rank {r}")


def test_batched_all_reduce_refuses_capture():
    R = 2
    ts = [[si.torch_tensor_for(9, t, R, r, (1000 + t,), device=DEV) for r in range(R)] for t in range(3)]
    outs = [[torch.empty_like(x) for x in per] for per in ts]
    with session(R, device=0):
        rr.all_reduce_many(ts, "mean", out=outs)  # fine outside a capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(rr.CollectiveError) as ei:
            with torch.cuda.graph(g):
                rr.all_reduce_many(ts, "mean", out=outs)
        assert ei.value.code == rr.RC_ERR_INVALID_ARGUMENT
        assert "graph" in str(ei.value)
        torch.cuda.synchronize()
        # the session and the stream are still usable
        got = rr.all_reduce_many(ts, "mean")
        torch.cuda.synchronize()
        for t in range(3):
            want = oracle.all_reduce_closed_form([host(x) for x in ts[t]], "mean")
            assert_bits(host(got[t][0]), want, f"tensor {t} after the refused capture")


def test_static_batched_all_reduce_replays():
    """rc_all_reduce_many_static captured into a graph: its table writes are
    kernels whose words travel in the kernel arguments, so each replay
    rewrites the static scratch before the batched fold reads it, even after
    eager static calls of another batch have left their own tables there."""
    R = 4
    shapes = [(2048, 4096), (4096,), (4096,), (1000,), (257,), (3,), ()]  # the first gets its own launch
    other = [(513,), (2048,), (9,)]

    def make(shps, seed):
        return [[si.torch_tensor_for(seed, t, R, r, s, device=DEV) for r in range(R)] for t, s in enumerate(shps)]

    ts = make(shapes, 740)
    outs = [[torch.empty_like(x) for x in per] for per in ts]
    ots = make(other, 741)
    with session(R, device=0):
        rr.all_reduce_many_static(ts, "mean", out=outs)  # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rr.all_reduce_many_static(ts, "mean", out=outs)
        for rep in range(4):
            fresh = make(shapes, 750 + rep)
            for per, fper in zip(ts, fresh):
                for x, f in zip(per, fper):
                    x.copy_(f)
            # eager static call of another batch: its tables overwrite the scratch
            got_other = rr.all_reduce_many_static(ots, "sum")
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            eager = rr.all_reduce_many(ts, "mean")
            torch.cuda.synchronize()
            for t in range(len(shapes)):
                for r in range(R):
                    assert torch.equal(outs[t][r].view(torch.int32), eager[t][r].view(torch.int32)), (
                        f"replay {rep} tensor {t} rank {r} differs from the eager batch")
            for t in (0, 3, len(shapes) - 1):
                hx = [host(x).reshape(-1) for x in ts[t]]
                assert_bits(host(outs[t][rep % R]).reshape(-1), oracle.all_reduce(hx, "mean")[0],
                            f"replay {rep} tensor {t} vs oracle")
            hx = [host(x).reshape(-1) for x in ots[1]]
            assert_bits(host(got_other[1][0]).reshape(-1), oracle.all_reduce(hx, "sum")[0], f"other batch {rep}")
