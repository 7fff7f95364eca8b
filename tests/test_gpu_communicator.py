"""The Communicator class on the GPU, used as the monarch Communicator page
describes: each logical rank builds its own communicator on its own thread and
calls every method with its own tensor and stream.  Results against the CPU
oracle."""

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


def test_every_method_from_rank_threads():
    R = 4
    M = 100_003
    N = R * M
    xs = si.torch_rank_inputs(R, N, "f32", "normal", 800, device=DEV)
    torch.cuda.synchronize()
    hx = [host(x) for x in xs]
    streams = [torch.cuda.Stream() for _ in range(R)]
    errs = []
    res = [dict() for _ in range(R)]

    def rank(r):
        try:
            comm = rr.Communicator(r, R, device=0)
            s = streams[r]
            out = res[r]
            with torch.cuda.stream(s):
                t = xs[r].clone()
                comm.all_reduce(t, "sum", stream=s)               # in place
                out["all_reduce"] = t
                b = xs[r].clone()
                comm.broadcast(b, 2, stream=s)
                out["broadcast"] = b
                d = xs[r].clone()
                comm.reduce(d, "max", 1, stream=s)                # in place at the root
                out["reduce"] = d
                lst = [torch.empty(M, device=DEV) for _ in range(R)]
                comm.all_gather(lst, xs[r][:M].contiguous(), stream=s)
                out["all_gather"] = lst
                big = torch.empty(N, device=DEV)
                comm.all_gather_into_tensor(big, xs[r][:M].contiguous(), stream=s)
                out["all_gather_into_tensor"] = big
                sh = torch.empty(M, device=DEV)
                comm.reduce_scatter_tensor(sh, xs[r], "sum", stream=s)
                out["reduce_scatter_tensor"] = sh
                a2a = torch.empty(N, device=DEV)
                comm.all_to_all_single(a2a, xs[r], stream=s)
                out["all_to_all_single"] = a2a
                got = torch.empty(M, device=DEV)
                if r % 2 == 0:
                    comm.send(xs[r][:M].contiguous(), (r + 1) % R, stream=s)
                    comm.recv(got, (r - 1) % R, stream=s)
                else:
                    comm.recv(got, (r - 1) % R, stream=s)
                    comm.send(xs[r][:M].contiguous(), (r + 1) % R, stream=s)
                out["p2p"] = got
                comm.barrier(stream=s)
                sub = comm.split_from([2, 0] if r % 2 == 0 else [])
                if sub is not None:
                    assert sub.world_size == 2 and sub.rank == [2, 0].index(r)
                    u = xs[r].clone()
                    sub.all_reduce(u, "sum", stream=s)
                    out["sub"] = u
                    sub.finish()
            s.synchronize()
            comm.finish()
        except BaseException as e:  # noqa: BLE001
            errs.append(e)

    ts = [threading.Thread(target=rank, args=(r,)) for r in range(R)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not errs, errs
    torch.cuda.synchronize()
    want_ar = oracle.all_reduce_closed_form(hx, "sum")
    want_red = oracle.reduce(hx, 1, "max")[1]
    want_rs = oracle.reduce_scatter(hx, "sum")
    want_a2a = oracle.all_to_all_single(hx)
    shards = [h[:M] for h in hx]
    want_sub = oracle.all_reduce_closed_form([hx[2], hx[0]], "sum")
    for r in range(R):
        o = res[r]
        assert_bits(host(o["all_reduce"]), want_ar, f"all_reduce rank {r}")
        assert_bits(host(o["broadcast"]), hx[2], f"broadcast rank {r}")
        assert_bits(host(o["reduce"]), want_red if r == 1 else hx[r], f"reduce rank {r}")
        for k in range(R):
            assert_bits(host(o["all_gather"][k]), shards[k], f"all_gather rank {r} shard {k}")
        assert_bits(host(o["all_gather_into_tensor"]), np.concatenate(shards), f"all_gather_into_tensor rank {r}")
        assert_bits(host(o["reduce_scatter_tensor"]), want_rs[r], f"reduce_scatter_tensor rank {r}")
        assert_bits(host(o["all_to_all_single"]), want_a2a[r], f"all_to_all_single rank {r}")
        assert_bits(host(o["p2p"]), shards[(r - 1) % R], f"send/recv rank {r}")
        if r % 2 == 0:
            assert_bits(host(o["sub"]), want_sub, f"split group rank {r}")
        else:
            assert "sub" not in o
