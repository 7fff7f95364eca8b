"""rc_all_reduce_many_static, the allocation-free batched all-reduce, against
rc_all_reduce_many through the C ABI: the same tensors, bit for bit, on two
calls in a row (the second with a smaller input, so stale tables from the
first would show), a session of another rank count, views off the 16-byte
grid, and a batch whose tables exceed the static scratch (refused before
anything is written).  The oracle checks the static path's outputs too."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import assert_bits, host, session

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tensors_of(R, shapes, seed, offsets=None):
    """ts[t][r]: rank r's tensor t, N(0,1) from its own seed; offsets[t] > 0
    makes every rank's tensor t a view that many elements into a larger one."""
    ts = []
    for t, shp in enumerate(shapes):
        per = []
        for r in range(R):
            n = int(np.prod(shp)) if shp else 1
            off = offsets[t] if offsets else 0
            base = si.torch_tensor_for(seed, t, R, r, (n + off,), device=DEV)
            per.append(base[off:].view(shp))
        ts.append(per)
    return ts


def call(fn, ts, op, fill=float("nan")):
    """Run one rc_* batched entry point through the C ABI; returns (status, outputs)."""
    outs = [[torch.full_like(x, fill) for x in per] for per in ts]
    arr = rr.batch_bufs(ts, outs, rr.OPS[op])
    stream = torch.cuda.current_stream().cuda_stream
    rc = fn(len(ts), ctypes.c_void_p(arr.ctypes.data), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    return rc, outs


def same_bits(a, b, what):
    for t, (pa, pb) in enumerate(zip(a, b)):
        for r, (x, y) in enumerate(zip(pa, pb)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{what}: tensor {t} rank {r} differs"


def test_static_matches_arena_path_two_calls():
    lib = rr.library()
    R = 4
    # call 1: a tensor with a launch of its own (256 MiB of traffic), 40 that
    # share the batched launch, ragged and tiny ones
    shapes1 = [(2048, 4096)] + [(4096,)] * 40 + [(1000,), (257,), (3,), (1,), (65, 7), ()]
    # call 2: fewer and smaller tensors
    shapes2 = [(300,), (17,), (4096,), (5,)]
    with session(R):
        ts1 = tensors_of(R, shapes1, 11)
        rc, want1 = call(lib.rc_all_reduce_many, ts1, "mean")
        assert rc == rr.RC_OK, lib.rc_last_error().decode()
        rc, got1 = call(lib.rc_all_reduce_many_static, ts1, "mean")
        assert rc == rr.RC_OK, lib.rc_last_error().decode()
        same_bits(got1, want1, "first call")
        for t in (0, 1, 41, 42, 43, 46):
            hx = [host(x).reshape(-1) for x in ts1[t]]
            assert_bits(host(got1[t][t % R]), oracle.all_reduce(hx, "mean")[0], f"first call tensor {t} vs oracle")
        ts2 = tensors_of(R, shapes2, 12)
        rc, want2 = call(lib.rc_all_reduce_many, ts2, "sum")
        assert rc == rr.RC_OK, lib.rc_last_error().decode()
        rc, got2 = call(lib.rc_all_reduce_many_static, ts2, "sum")
        assert rc == rr.RC_OK, lib.rc_last_error().decode()
        same_bits(got2, want2, "second call")
        for t in range(len(shapes2)):
            hx = [host(x).reshape(-1) for x in ts2[t]]
            assert_bits(host(got2[t][0]), oracle.all_reduce(hx, "sum")[0], f"second call tensor {t} vs oracle")
        # the first call's outputs are untouched by the second
        rc, again1 = call(lib.rc_all_reduce_many, ts1, "mean")
        same_bits(got1, again1, "first call's outputs after the second")


def test_static_other_rank_count_and_offsets():
    lib = rr.library()
    R = 8
    shapes = [(4096,)] * 6 + [(1031,), (8,), (2, 3, 5)]
    offsets = [0, 1, 2, 3, 0, 1, 3, 2, 1]
    with session(R):
        ts = tensors_of(R, shapes, 13, offsets)
        for op in ("sum", "max"):
            rc, want = call(lib.rc_all_reduce_many, ts, op)
            assert rc == rr.RC_OK, lib.rc_last_error().decode()
            rc, got = call(lib.rc_all_reduce_many_static, ts, op)
            assert rc == rr.RC_OK, lib.rc_last_error().decode()
            same_bits(got, want, f"8 ranks {op}")
            hx = [host(x).reshape(-1) for x in ts[6]]
            assert_bits(host(got[6][5]), oracle.all_reduce(hx, op)[0], f"8 ranks {op} vs oracle")


def test_static_refuses_tables_beyond_scratch():
    lib = rr.library()
    R = 16
    # 300 tensors x 16 segments of 280 bytes of descriptors: past 1 MiB
    shapes = [(64,)] * 300
    with session(R):
        ts = tensors_of(R, shapes, 14)
        rc, outs = call(lib.rc_all_reduce_many_static, ts, "sum", fill=-1.0)
        assert rc == rr.RC_ERR_INVALID_ARGUMENT
        assert "static scratch" in lib.rc_last_error().decode()
        for per in outs[:3] + outs[-3:]:
            for o in per:
                assert torch.all(o == -1.0).item(), "an output was written by a refused call"
        # the session is still usable, and a batch that fits runs
        rc, got = call(lib.rc_all_reduce_many_static, ts[:100], "sum")
        assert rc == rr.RC_OK, lib.rc_last_error().decode()
        rc, want = call(lib.rc_all_reduce_many, ts[:100], "sum")
        same_bits(got, want, "100 tensors at 16 ranks")
