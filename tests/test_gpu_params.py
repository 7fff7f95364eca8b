"""The parameter-keyed gradient sync on the GPU, bit for bit against the CPU
oracle's all_reduce_params: per-rank maps listed in different orders, empty
and scalar parameters, a parameter large enough for a launch of its own, in
place, from one thread and from one thread per rank."""

import random
import threading

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import SENTINEL, assert_bits, host, session

pytestmark = pytest.mark.gpu
DEV = "cuda"

# parameter id -> shape: several tiles, ragged tails, empty, scalar
SMALL = {101: (512, 33), 7: (257,), 9000: (0,), 3: (), 42: (4096,), 5: (3, 1000, 7), 77: (65_537,)}


def make_maps(R, specs, seed, sigma=1e-3):
    """R maps {id: tensor}, each rank listing its IDs in its own order."""
    maps = []
    for r in range(R):
        keys = list(specs)
        random.Random(seed * 31 + r).shuffle(keys)
        maps.append({k: si.torch_tensor_for(seed, k, R, r, specs[k], device=DEV) for k in keys})
    return maps


def host_maps(maps):
    return [{k: host(v) for k, v in m.items()} for m in maps]


def check(got, want, what):
    for r, (g, w) in enumerate(zip(got, want)):
        assert set(g) == set(w), f"{what}: rank {r} IDs"
        for k in w:
            assert_bits(host(g[k]), w[k], f"{what}: rank {r} parameter {k}")


@pytest.mark.parametrize("R", [1, 2, 4, 8])
@pytest.mark.parametrize("op", ["mean", "sum"])
def test_params_whole_call(R, op):
    maps = make_maps(R, SMALL, seed=50 + R)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), op)
    with session(R, device=0):
        got = rr.all_reduce_params(maps, op)
        torch.cuda.synchronize()
    check(got, want, f"R={R} {op}")


def test_params_with_own_launch_tensor_and_in_place():
    """A 64 MiB parameter takes its own fold launch, the rest share the
    batched launch; in place (out = grads) as an optimizer would use it."""
    R = 4
    specs = dict(SMALL)
    specs[1 << 40] = (4096, 4096)  # 64 MiB per rank
    maps = make_maps(R, specs, seed=61)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "mean")
    with session(R, device=0):
        rr.all_reduce_params(maps, "mean", out=maps)
        torch.cuda.synchronize()
    check(maps, want, "in place")


def test_params_mismatch_touches_nothing():
    R = 3
    maps = make_maps(R, SMALL, seed=62)
    del maps[1][42]
    outs = [{k: torch.full(v.shape, SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
             for k, v in m.items()} for m in maps]
    with session(R, device=0):
        with pytest.raises(rr.CollectiveError) as ei:
            rr.all_reduce_params(maps, "mean", out=outs)
        assert ei.value.code == rr.RC_ERR_PARAM_MISMATCH
        torch.cuda.synchronize()
    for m in outs:
        for v in m.values():
            assert torch.all(v.view(torch.int32) == SENTINEL).item()


@pytest.mark.parametrize("n_streams", [1, 4])
def test_params_rank_threads(n_streams):
    """The pages' calling pattern: each rank's thread syncs its own map on
    its own stream; the producer runs right before the call and the
    consumer right after, with no host synchronisation."""
    R = 4
    maps = make_maps(R, SMALL, seed=63 + n_streams)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "mean")
    pool = [torch.cuda.Stream() for _ in range(n_streams)]
    for r in range(R):
        rr.rank_register(r, R, device=0)
    errs = []
    got = [None] * R

    def rank(r):
        try:
            s = pool[r % n_streams]
            with torch.cuda.stream(s):
                grads = {k: (v * 2.0 - v) / 1.0 for k, v in maps[r].items()}  # exact copy, on s
                out = rr.rank_all_reduce_params(r, grads, "mean", stream=s)
                got[r] = {k: v.clone() for k, v in out.items()}
                for v in grads.values():
                    v.mul_(0)
        except BaseException as e:  # noqa: BLE001
            errs.append(e)

    try:
        ts = [threading.Thread(target=rank, args=(r,)) for r in range(R)]
        for t in ts:
            t.start()
        for t in ts:
            t.join(timeout=120)
        assert not errs, errs
        torch.cuda.synchronize()
        check(got, want, f"rank threads, {n_streams} streams")
    finally:
        for r in range(R):
            rr.rank_finish(r)


def test_params_equal_all_reduce_many_bits():
    """The same tensors through all_reduce_many in ID order give the same bits."""
    R = 4
    maps = make_maps(R, SMALL, seed=64)
    order = sorted(SMALL)
    with session(R, device=0):
        a = rr.all_reduce_params(maps, "mean")
        b = rr.all_reduce_many([[maps[r][k] for r in range(R)] for k in order], "mean")
        torch.cuda.synchronize()
    for t, k in enumerate(order):
        for r in range(R):
            assert torch.equal(a[r][k].view(-1).view(torch.int32), b[t][r].view(-1).view(torch.int32))
    assert np.all([set(m) == set(SMALL) for m in a])


# ---------------------------------------------------------------- accumulators

def make_accs(maps, ids, seed):
    """Per-rank accumulators for the parameters in ids (every rank)."""
    R = len(maps)
    return [{k: si.torch_tensor_for(seed, k, R, r, tuple(maps[r][k].shape), device=DEV) for k in ids}
            for r in range(R)]


@pytest.mark.parametrize("R", [2, 4, 8])
@pytest.mark.parametrize("op", ["mean", "sum"])
def test_params_accumulated(R, op):
    """Some parameters carry accumulators, some do not: the batch splits into
    an accumulating and a plain launch, and both match the oracle."""
    maps = make_maps(R, SMALL, seed=70 + R)
    accs = make_accs(maps, [101, 7, 3, 77], seed=90 + R)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), op, acc=host_maps(accs))
    with session(R, device=0):
        got = rr.all_reduce_params(maps, op, acc=accs)
        torch.cuda.synchronize()
    check(got, want, f"accumulated R={R} {op}")


@pytest.mark.parametrize("R", [2, 3, 8])
def test_params_accumulated_whole_tiles(R):
    """Parameters large enough for launches of their own whose ring segments
    are whole tiles (the whole-tile fold with accumulators) next to one that
    is not, for rank counts whose unroll differs from 4 ranks'."""
    seg = {2: 2**21, 3: 2**20, 8: 2**17}[R]  # elements per segment: whole tiles, 64 MiB+ moved
    specs = {11: (R * seg,), 12: (R, seg), 13: (R * seg + 5,), 14: (300,)}
    maps = make_maps(R, specs, seed=120 + R)
    accs = make_accs(maps, [11, 12, 13, 14], seed=130 + R)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "mean", acc=host_maps(accs))
    with session(R, device=0):
        got = rr.all_reduce_params(maps, "mean", acc=accs)
        torch.cuda.synchronize()
    check(got, want, f"accumulated whole tiles R={R}")


# elements per ring segment: whole tiles of every unroll, 64 MiB and more moved
ACC_TABLE_SEG = {1: 2**23, 2: 2**21, 3: 2**20, 4: 2**19, 5: 2**18, 6: 2**18, 7: 2**17, 8: 2**17, 9: 2**17}


@pytest.mark.parametrize("R,case", [(R, "f32_mean_in_place") for R in range(1, 10)] +
                         [(R, "i32_sum") for R in (1, 4, 7, 9)])
def test_params_accumulated_table_kernels(R, case):
    """Whole-tile folds with accumulators on their pointer-table kernel (up
    to 8 ranks: each operand's accumulator in the table row's upper half) and
    past it (9 ranks), for every rank count and so every unroll: float32 Mean
    written in place into the accumulators, int32 Sum into new outputs, next
    to a parameter that is not whole tiles."""
    seg = ACC_TABLE_SEG[R]
    specs = {21: (R * seg,), 22: (R * seg + 3,)}
    dtype = "i32" if case == "i32_sum" else "f32"
    op = "sum" if case == "i32_sum" else "mean"
    seed = 140 + R
    maps = [{k: si.torch_tensor_for(seed, k, R, r, specs[k], dtype=dtype, device=DEV) for k in specs}
            for r in range(R)]
    accs = [{k: si.torch_tensor_for(seed + 50, k, R, r, specs[k], dtype=dtype, device=DEV) for k in specs}
            for r in range(R)]
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), op, acc=host_maps(accs))
    with session(R, device=0):
        if case == "f32_mean_in_place":
            rr.all_reduce_params(maps, op, out=accs, acc=accs)
            got = accs
        else:
            got = rr.all_reduce_params(maps, op, acc=accs)
        torch.cuda.synchronize()
    check(got, want, f"accumulated table kernels R={R} {case}")


@pytest.mark.parametrize("algo", ["direct", "ring"])
def test_params_accumulated_own_launch_in_place(algo):
    """A parameter large enough for its own fold launch (direct, or the ring's
    two launches), written in place into the accumulators' storage."""
    R = 4
    specs = {5: (2_000_003,), 6: (1000,)}
    maps = make_maps(R, specs, seed=81)
    accs = make_accs(maps, [5, 6], seed=82)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "mean", acc=host_maps(accs))
    with session(R, device=0, algo=algo):
        rr.all_reduce_params(maps, "mean", out=accs, acc=accs)
        torch.cuda.synchronize()
    check(accs, want, f"accumulated own launch {algo}, in place")


def test_params_accumulated_i32_sum():
    R = 4
    specs = {1: (70_001,), 2: (33,)}
    maps = [{k: si.torch_tensor_for(83, k, R, r, specs[k], dtype="i32", device=DEV) for k in specs} for r in range(R)]
    accs = [{k: si.torch_tensor_for(84, k, R, r, specs[k], dtype="i32", device=DEV) for k in specs} for r in range(R)]
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "sum", acc=host_maps(accs))
    with session(R, device=0):
        got = rr.all_reduce_params(maps, "sum", acc=accs)
        torch.cuda.synchronize()
    check(got, want, "accumulated int32")


def test_fused_equals_accumulate_then_sync():
    """The fused pass gives the bits of adding the last microbatch with a
    separate elementwise add and then syncing."""
    R = 4
    maps = make_maps(R, SMALL, seed=85)
    accs = make_accs(maps, list(SMALL), seed=86)
    with session(R, device=0):
        fused = rr.all_reduce_params(maps, "mean", acc=accs)
        summed = [{k: accs[r][k] + maps[r][k] for k in SMALL} for r in range(R)]
        plain = rr.all_reduce_params(summed, "mean")
        torch.cuda.synchronize()
    for r in range(R):
        for k in SMALL:
            assert torch.equal(fused[r][k].view(-1).view(torch.int32), plain[r][k].view(-1).view(torch.int32)), k


def test_params_accumulated_rank_threads():
    R = 4
    maps = make_maps(R, SMALL, seed=87)
    accs = make_accs(maps, [101, 42, 77], seed=88)
    torch.cuda.synchronize()
    want = oracle.all_reduce_params(host_maps(maps), "mean", acc=host_maps(accs))
    pool = [torch.cuda.Stream() for _ in range(R)]
    for r in range(R):
        rr.rank_register(r, R, device=0)
    errs = []
    got = [None] * R

    def rank(r):
        try:
            with torch.cuda.stream(pool[r]):
                out = rr.rank_all_reduce_params(r, maps[r], "mean", stream=pool[r], acc=accs[r])
                got[r] = {k: v.clone() for k, v in out.items()}
        except BaseException as e:  # noqa: BLE001
            errs.append(e)

    try:
        ts = [threading.Thread(target=rank, args=(r,)) for r in range(R)]
        for t in ts:
            t.start()
        for t in ts:
            t.join(timeout=120)
        assert not errs, errs
        torch.cuda.synchronize()
        check(got, want, "accumulated, rank threads")
    finally:
        for r in range(R):
            rr.rank_finish(r)


@pytest.mark.parametrize("R", [2, 4])
def test_params_accumulated_misaligned_views(R):
    """Gradients and accumulators carved out of larger buffers at offsets of
    0-3 elements that differ between ranks: every job runs element by element
    (in rounds of several elements per lane), with and without accumulators,
    and the bits still equal the oracle's."""
    specs = {11: (40_003,), 12: (1_001,), 13: (5_000,)}
    grads, accs = [], []
    for r in range(R):
        g, a = {}, {}
        for k, shape in specs.items():
            n = shape[0]
            og, oa = (r + k) % 4, (r * 3 + k) % 4
            g[k] = si.torch_tensor_for(70, k, R, r, (n + 4,), device=DEV)[og:og + n]
            a[k] = si.torch_tensor_for(71, k, R, r, (n + 4,), device=DEV)[oa:oa + n]
        grads.append(g)
        accs.append(a)
    torch.cuda.synchronize()
    for use_acc in (False, True):
        want = oracle.all_reduce_params(host_maps(grads), "mean", acc=host_maps(accs) if use_acc else None)
        outs = []
        for r in range(R):
            outs.append({k: torch.empty(v.numel() + 4, device=DEV)[(r + 1) % 4:(r + 1) % 4 + v.numel()]
                         for k, v in grads[r].items()})
        with session(R, device=0):
            rr.all_reduce_params(grads, "mean", out=outs, acc=accs if use_acc else None)
            torch.cuda.synchronize()
        check(outs, want, f"R={R} acc={use_acc}")
