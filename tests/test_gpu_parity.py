"""GPU parity: every collective through the C ABI against the CPU oracle.

Sizes here are ones the oracle finishes in seconds; they span several tiles,
ragged tails, empty segments, misaligned views and every rank count.  The bar
is bit-exact equality (the oracle reproduces the library's documented ring
order), with the order-free tolerance checked as a second guard for float32.
"""

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import SENTINEL, assert_bits, assert_within_bound, host, sentinel_like, session

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gen(R, N, dtype="f32", dist="normal", seed=0):
    return si.torch_rank_inputs(R, N, dtype, dist, seed, device=DEV)


def sync():
    torch.cuda.synchronize()


def check_unchanged(xs, keep, what):
    for r, (x, k) in enumerate(zip(xs, keep)):
        assert_bits(host(x), k, f"{what}: input of rank {r} changed")


# ---------------------------------------------------------------- the pages' example

def test_pages_example_four_ranks_257_fp32():
    """ruCCL README, "CUDA tensor example": 4 logical ranks on GPU 0, 257 FP32
    elements, sum and mean on every rank, inputs unchanged; plus reduce to
    root 0 and broadcast from rank 1."""
    R, N = 4, 257
    xs = gen(R, N, "f32", "uniform", 0)
    hx = [host(x).copy() for x in xs]
    with session(R):
        for op in ("sum", "mean"):
            outs = rr.all_reduce(xs, op)
            sync()
            want = oracle.all_reduce(hx, op)
            for r in range(R):
                assert_bits(host(outs[r]), want[r], f"all_reduce {op} rank {r}")
            assert_within_bound(host(outs[0]), hx, op, f"all_reduce {op}")
        out = [sentinel_like(torch, x) for x in xs]
        rr.reduce(xs, 0, "sum", out=out)
        sync()
        want = oracle.reduce(hx, 0, "sum")
        assert_bits(host(out[0]), want[0], "reduce root 0")
        for r in range(1, R):
            assert np.all(host(out[r]).view(np.uint32) == SENTINEL), f"non-root {r} written"
        sends = [None, xs[1], None, None]
        outs = rr.broadcast(sends)
        sync()
        want = oracle.broadcast([None, hx[1], None, None])
        for r in (0, 2, 3):
            assert_bits(host(outs[r]), want[r], f"broadcast rank {r}")
    check_unchanged(xs, hx, "example")


# ---------------------------------------------------------------- all_reduce sweep

SIZES = [0, 1, 3, 5, 8, 65, 257, 1023, 4099, 50_001, 200_003]
RANKS = [1, 2, 3, 4, 5, 7, 8, 12, 16]
OPS = [("f32", "sum"), ("f32", "mean"), ("f32", "max"), ("i32", "sum"), ("i32", "max")]


@pytest.mark.parametrize("R", RANKS)
@pytest.mark.parametrize("dtype,op", OPS)
@pytest.mark.parametrize("algo", ["direct", "ring"])
def test_all_reduce_sweep(R, dtype, op, algo):
    with session(R, algo=algo):
        for i, N in enumerate(SIZES):
            dist = "int" if dtype == "i32" else "normal"
            xs = gen(R, N, dtype, dist, seed=1000 * R + i)
            hx = [host(x).copy() for x in xs]
            outs = rr.all_reduce(xs, op)
            sync()
            want = oracle.all_reduce_closed_form(hx, op)
            for r in range(R):
                assert_bits(host(outs[r]), want, f"R={R} N={N} {dtype} {op} {algo} rank {r}")
            if dtype == "f32" and op != "max":
                assert_within_bound(host(outs[0]), hx, op, f"R={R} N={N} {op}")
            check_unchanged(xs, hx, f"R={R} N={N}")


@pytest.mark.parametrize("R", sorted(set(RANKS) | {6}))
@pytest.mark.parametrize("dtype,op", OPS)
def test_whole_tile_collectives(R, dtype, op):
    """Sizes whose ring segments are whole tiles on 256-byte boundaries (every
    unroll the ranks use): all_reduce (direct and ring), reduce, reduce_scatter,
    all_gather and broadcast run the whole-tile kernels; bits against the
    oracle, inputs unchanged."""
    N = R * 8192  # a multiple of 256 * U elements per segment for every U
    dist = "int" if dtype == "i32" else "normal"
    xs = gen(R, N, dtype, dist, seed=4000 + 10 * R + OPS.index((dtype, op)))
    hx = [host(x).copy() for x in xs]
    want = oracle.all_reduce_closed_form(hx, op)
    for algo in ("direct", "ring"):
        with session(R, algo=algo):
            outs = rr.all_reduce(xs, op)
            sync()
            for r in range(R):
                assert_bits(host(outs[r]), want, f"all_reduce {algo} R={R} {dtype} {op} rank {r}")
    with session(R):
        root = R // 2
        red = rr.reduce(xs, root, op)
        shards = rr.reduce_scatter(xs, op)
        sync()
        assert_bits(host(red[root]), want, f"reduce R={R} {dtype} {op}")
        for r in range(R):
            assert_bits(host(shards[r]), want[r * 8192:(r + 1) * 8192], f"reduce_scatter R={R} {op} rank {r}")
        gathered = rr.all_gather(shards)
        sends = [xs[r] if r == R - 1 else None for r in range(R)]
        bc = rr.broadcast(sends)
        sync()
        for r in range(R):
            assert_bits(host(gathered[r]), want, f"all_gather R={R} {op} rank {r}")
            if r != R - 1:  # the sender's own output is not asked for
                assert_bits(host(bc[r]), hx[R - 1], f"broadcast R={R} rank {r}")
    check_unchanged(xs, hx, f"whole tiles R={R}")


@pytest.mark.parametrize("R", [2, 4, 8])
def test_all_reduce_matches_ring_simulation(R):
    """The closed form used above equals the oracle's message-by-message ring."""
    with session(R):
        for N in (7, 257, 4099, 50_001):
            xs = gen(R, N, "f32", "normal", seed=77 + N)
            hx = [host(x) for x in xs]
            for op in ("sum", "mean"):
                outs = rr.all_reduce(xs, op)
                sync()
                want = oracle.all_reduce(hx, op)
                for r in range(R):
                    assert_bits(host(outs[r]), want[r], f"ring sim R={R} N={N} {op} rank {r}")


@pytest.mark.parametrize("R", [3, 4, 8])
def test_all_reduce_misaligned_views(R):
    """Views starting 1-3 elements past a 16-byte boundary: the same offset on
    every rank (scalar head, vector body) and different offsets per rank
    (element-by-element path)."""
    N = 50_003
    with session(R):
        for offsets in ([1] * R, [2] * R, [3] * R, [r % 4 for r in range(R)], [(r * 3 + 1) % 4 for r in range(R)]):
            bases = gen(R, N + 8, "f32", "normal", seed=sum(offsets) + R)
            xs = [b[o:o + N] for b, o in zip(bases, offsets)]
            obases = [torch.empty(N + 8, dtype=torch.float32, device=DEV) for _ in range(R)]
            outs = [b[(o + 1) % 4:(o + 1) % 4 + N] for b, o in zip(obases, offsets)]
            hx = [host(x).copy() for x in xs]
            for op in ("sum", "mean", "max"):
                rr.all_reduce(xs, op, out=outs)
                sync()
                want = oracle.all_reduce_closed_form(hx, op)
                for r in range(R):
                    assert_bits(host(outs[r]), want, f"offsets {offsets} {op} rank {r}")


@pytest.mark.parametrize("R", [2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("dtype,op", OPS)
def test_whole_tile_outputs_off_bursts(R, dtype, op):
    """Whole-tile folds whose outputs start 1-15 elements past a 64-byte
    boundary (inputs aligned, so the jobs stay whole tiles): the shifted
    kernel writes each such output over burst-aligned ranges, reaching back
    up to 15 elements into the previous tile's range and writing a job's
    last elements from its last tile.  all_reduce (direct and ring), reduce
    to one root and reduce_scatter, with every byte around the outputs
    holding a sentinel that must survive; in place runs the unshifted
    kernel.  Bits against the oracle."""
    N = R * 8192  # whole tiles of every unroll, several per segment
    M = N // R
    PAD = 32
    offs = [(5 * r) % 16 for r in range(R)]  # rank 0 on a boundary: the aligned class stays the heaviest
    dist = "int" if dtype == "i32" else "normal"
    seed = 4500 + 10 * R + OPS.index((dtype, op))
    xs = gen(R, N, dtype, dist, seed=seed)
    hx = [host(x).copy() for x in xs]
    want = oracle.all_reduce_closed_form(hx, op)

    def padded(n):
        bases = [sentinel_like(torch, torch.empty(n + PAD, dtype=xs[0].dtype, device=DEV)) for _ in range(R)]
        return bases, [b[o:o + n] for b, o in zip(bases, offs)]

    def check_pads(bases, n, what, written=None):
        for r, (b, o) in enumerate(zip(bases, offs)):
            hb = host(b).view(np.uint32)
            if written is not None and r not in written:
                assert np.all(hb == SENTINEL), f"{what}: rank {r} written"
                continue
            assert np.all(hb[:o] == SENTINEL) and np.all(hb[o + n:] == SENTINEL), \
                f"{what}: rank {r} written outside its output (offset {o})"

    for algo in ("direct", "ring"):
        with session(R, algo=algo):
            bases, outs = padded(N)
            rr.all_reduce(xs, op, out=outs)
            sync()
            for r in range(R):
                assert_bits(host(outs[r]), want, f"all_reduce {algo} R={R} {dtype} {op} rank {r}")
            check_pads(bases, N, f"all_reduce {algo}")
    with session(R):
        root = R - 1
        bases, outs = padded(N)
        rr.reduce(xs, root, op, out=[o if r == root else None for r, o in enumerate(outs)])
        sync()
        assert_bits(host(outs[root]), want, f"reduce R={R} {dtype} {op}")
        check_pads(bases, N, "reduce", written={root})
        bases, shards = padded(M)
        rr.reduce_scatter(xs, op, out=shards)
        sync()
        for r in range(R):
            assert_bits(host(shards[r]), want[r * M:(r + 1) * M], f"reduce_scatter R={R} {op} rank {r}")
        check_pads(bases, M, "reduce_scatter")
        # in place at the same offsets: the unshifted kernel
        bases, views = padded(N)
        for v, x in zip(views, xs):
            v.copy_(x)
        rr.all_reduce(views, op, out=views)
        sync()
        for r in range(R):
            assert_bits(host(views[r]), want, f"in place R={R} {op} rank {r}")
        check_pads(bases, N, "in place")
    check_unchanged(xs, hx, f"outputs off bursts R={R}")


def test_all_reduce_in_place():
    R, N = 8, 200_003
    with session(R):
        for op in ("sum", "mean", "max"):
            xs = gen(R, N, "f32", "normal", seed=5)
            hx = [host(x).copy() for x in xs]
            rr.all_reduce(xs, op, out=xs)
            sync()
            want = oracle.all_reduce_closed_form(hx, op)
            for r in range(R):
                assert_bits(host(xs[r]), want, f"in place {op} rank {r}")


def test_schedule_invariance():
    """The bits do not depend on tile size, grid, cache hint or algorithm."""
    R, N = 8, 200_003
    xs = gen(R, N, "f32", "normal", seed=9)
    hx = [host(x) for x in xs]
    want = {op: oracle.all_reduce_closed_form(hx, op) for op in ("sum", "mean")}
    for cfg in (dict(), dict(tile_elems=4096), dict(tile_elems=16384), dict(max_workgroups=1),
                dict(max_workgroups=7), dict(cache_hint="normal"), dict(algo="ring", tile_elems=8192),
                dict(algo="ring", max_workgroups=3)):
        with session(R, **cfg):
            for op in ("sum", "mean"):
                outs = rr.all_reduce(xs, op)
                sync()
                for r in range(R):
                    assert_bits(host(outs[r]), want[op], f"{cfg} {op} rank {r}")


def test_schedule_invariance_whole_tiles():
    """At a whole-tile size the default launch runs the whole-tile kernels
    (non-temporal or, with cache_hint normal, cached accesses), larger tiles
    or a workgroup cap the general ones: the same bits from each."""
    R, N = 8, 8 * 65536
    xs = gen(R, N, "f32", "normal", seed=19)
    hx = [host(x) for x in xs]
    want = {op: oracle.all_reduce_closed_form(hx, op) for op in ("sum", "mean", "max")}
    for cfg in (dict(), dict(cache_hint="normal"), dict(tile_elems=4096), dict(max_workgroups=7),
                dict(algo="ring"), dict(algo="ring", cache_hint="normal"), dict(waves_per_cu=3)):
        with session(R, **cfg):
            for op in ("sum", "mean", "max"):
                outs = rr.all_reduce(xs, op)
                sync()
                for r in range(R):
                    assert_bits(host(outs[r]), want[op], f"{cfg} {op} rank {r}")


def test_special_values():
    """Subnormals are kept (no flush to zero); Max follows the NaN and signed
    zero rules."""
    R = 4
    tiny = np.float32(2.0 ** -149)
    rng = np.random.default_rng(3)
    ks = [rng.integers(-1000, 1001, size=4099) for _ in range(R)]
    hx = [(k.astype(np.float32) * tiny).astype(np.float32) for k in ks]
    xs = [torch.from_numpy(h).to(DEV) for h in hx]
    special = np.array([1.0, 0.0, -0.0, -0.0, np.nan, -np.inf, np.inf, 3.5], dtype=np.float32)
    hm = [np.tile(special, 37) for _ in range(R)]
    hm[2] = np.roll(hm[2], 1)
    hm[1] = hm[1].copy()
    hm[1][hm[1] == 0] = -0.0
    xm = [torch.from_numpy(h).to(DEV) for h in hm]
    with session(R):
        for op in ("sum", "mean"):
            outs = rr.all_reduce(xs, op)
            sync()
            assert_bits(host(outs[3]), oracle.all_reduce_closed_form(hx, op), f"subnormal {op}")
        outs = rr.all_reduce(xm, "max")
        sync()
        assert_bits(host(outs[0]), oracle.all_reduce_closed_form(hm, "max"), "max specials")
        outs = rr.all_reduce(xm, "sum")
        sync()
        got = host(outs[0])
        want = oracle.all_reduce_closed_form(hm, "sum")
        # NaN payloads of sums are the hardware's; compare NaN-ness, bits elsewhere
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert_bits(got[~nan], want[~nan], "sum specials")


# ---------------------------------------------------------------- reduce

@pytest.mark.parametrize("R", [1, 2, 4, 7, 8, 16])
def test_reduce_every_root(R):
    with session(R):
        for N in (1, 257, 50_001):
            xs = gen(R, N, "f32", "normal", seed=R + N)
            hx = [host(x).copy() for x in xs]
            for root in range(R):
                out = [sentinel_like(torch, x) for x in xs]
                rr.reduce(xs, root, "sum", out=out)
                sync()
                want = oracle.reduce(hx, root, "sum")
                assert_bits(host(out[root]), want[root], f"R={R} N={N} root {root}")
                assert_bits(host(out[root]), oracle.all_reduce_closed_form(hx, "sum"), "root == all_reduce")
                for r in range(R):
                    if r != root:
                        assert np.all(host(out[r]).view(np.uint32) == SENTINEL), f"non-root {r} written"
            check_unchanged(xs, hx, "reduce")


def test_reduce_i32_and_in_place_root():
    R, N = 4, 100_003
    xs = gen(R, N, "i32", "int", seed=21)
    hx = [host(x).copy() for x in xs]
    with session(R):
        for op in ("sum", "max"):
            out = rr.reduce(xs, 2, op)
            sync()
            assert_bits(host(out[2]), oracle.reduce(hx, 2, op)[2], f"i32 reduce {op}")
        ys = [x.clone() for x in xs]
        rr.reduce(ys, 1, "sum", out=[None, ys[1], None, None])
        sync()
        assert_bits(host(ys[1]), oracle.reduce(hx, 1, "sum")[1], "in place root")
        for r in (0, 2, 3):
            assert_bits(host(ys[r]), hx[r], f"non-root {r} in place untouched")


# ---------------------------------------------------------------- broadcast

@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
def test_broadcast_every_sender(R):
    with session(R):
        for N in (1, 5, 257, 50_001):
            src = gen(1, N, "i32", "int", seed=N)[0]
            for s in range(R):
                sends = [None] * R
                sends[s] = src
                outs = [torch.empty_like(src) for _ in range(R)]  # sender's recv written too
                rr.broadcast(sends, out=outs)
                sync()
                want = oracle.broadcast([host(src) if r == s else None for r in range(R)])
                for r in range(R):
                    assert_bits(host(outs[r]), want[r], f"R={R} N={N} sender {s} rank {r}")
                # sender passes no recv: receivers only
                outs = [None if r == s else torch.empty_like(src) for r in range(R)]
                rr.broadcast(sends, out=outs)
                sync()
                for r in range(R):
                    if r != s:
                        assert_bits(host(outs[r]), want[r], "receivers only")


def test_broadcast_in_place_sender_and_root_field():
    R, N = 4, 4099
    src = gen(1, N, "f32", "normal", seed=4)[0]
    keep = host(src).copy()
    with session(R):
        outs = [torch.empty_like(src) for _ in range(R)]
        outs[3] = src  # sender's recv == send: not rewritten
        rr.broadcast([None, None, None, src], out=outs, root=3)
        sync()
        for r in range(R):
            assert_bits(host(outs[r]), keep, f"rank {r}")
        with pytest.raises(rr.CollectiveError) as e:
            rr.broadcast([None, None, None, src], out=outs, root=1)
        assert e.value.code == rr.RC_ERR_ROOT_MISMATCH


# ---------------------------------------------------------------- reduce_scatter / all_gather

@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
def test_reduce_scatter_all_gather(R):
    with session(R):
        for M in (1, 5, 64, 1000, 12_345):
            for dtype, op in (("f32", "sum"), ("f32", "mean"), ("i32", "max")):
                xs = gen(R, R * M, dtype, "int" if dtype == "i32" else "normal", seed=R * M)
                hx = [host(x).copy() for x in xs]
                shards = rr.reduce_scatter(xs, op)
                sync()
                want = oracle.reduce_scatter(hx, op)
                for r in range(R):
                    assert_bits(host(shards[r]), want[r], f"RS R={R} M={M} {op} rank {r}")
                gathered = rr.all_gather(shards)
                sync()
                want_ag = oracle.all_gather([host(s) for s in shards])
                ar = oracle.all_reduce_closed_form(hx, op)
                for r in range(R):
                    assert_bits(host(gathered[r]), want_ag[r], f"AG rank {r}")
                    assert_bits(host(gathered[r]), ar, "AG(RS(x)) == AR(x)")
                check_unchanged(xs, hx, "RS")


def test_reduce_scatter_all_gather_in_place():
    """In place as recv_r = send_r + r*M (reduce_scatter) and send_r = recv_r +
    r*M (all_gather)."""
    R, M = 8, 10_007
    xs = gen(R, R * M, "f32", "normal", seed=8)
    hx = [host(x).copy() for x in xs]
    with session(R):
        bufs = [x.clone() for x in xs]
        rr.reduce_scatter(bufs, "sum", out=[b[r * M:(r + 1) * M] for r, b in enumerate(bufs)])
        sync()
        want = oracle.reduce_scatter(hx, "sum")
        for r in range(R):
            assert_bits(host(bufs[r][r * M:(r + 1) * M]), want[r], f"RS in place rank {r}")
        rr.all_gather([b[r * M:(r + 1) * M] for r, b in enumerate(bufs)], out=bufs)
        sync()
        ar = oracle.all_reduce_closed_form(hx, "sum")
        for r in range(R):
            assert_bits(host(bufs[r]), ar, f"AG in place rank {r}")


def test_all_gather_misaligned_shards():
    R, M = 4, 1001  # shard offsets k*M break 16-byte alignment of the outputs
    shards = gen(R, M, "i32", "int", seed=11)
    with session(R):
        outs = rr.all_gather(shards)
        sync()
        want = oracle.all_gather([host(s) for s in shards])
        for r in range(R):
            assert_bits(host(outs[r]), want[r], f"rank {r}")


# ---------------------------------------------------------------- batched

def _batch(R, shapes, seed, dtype="f32"):
    out = []
    for t, shp in enumerate(shapes):
        per = []
        for r in range(R):
            g = torch.Generator(device=DEV).manual_seed(seed * 1000 + t * R + r)
            if dtype == "f32":
                per.append(torch.randn(shp, generator=g, device=DEV) * 1e-3)
            else:
                per.append(torch.randint(-2 ** 20, 2 ** 20, shp, generator=g, device=DEV, dtype=torch.int32))
        out.append(per)
    return out


SHAPES = [(5,), (), (0,), (257,), (64, 33), (4096,), (100_003,), (3, 0, 2), (1,), (2048, 3)]


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype,op", [("f32", "mean"), ("f32", "sum"), ("f32", "max"), ("i32", "sum")])
def test_all_reduce_many(R, dtype, op):
    tensors = _batch(R, SHAPES, seed=R, dtype=dtype)
    with session(R):
        outs = rr.all_reduce_many(tensors, op)
        sync()
        for t, per in enumerate(tensors):
            hx = [host(x) for x in per]
            want = oracle.all_reduce(hx, op)
            single = rr.all_reduce(per, op)
            sync()
            for r in range(R):
                assert_bits(host(outs[t][r]), want[r], f"tensor {t} {SHAPES[t]} rank {r}")
                assert_bits(host(single[r]), host(outs[t][r]), f"batched == single, tensor {t}")


@pytest.mark.parametrize("R", [2, 4, 8])
def test_all_reduce_many_mixed_sizes(R):
    """Large tensors run as launches of their own and small ones in one batched
    launch; both kinds in one call, every tensor equal to the oracle."""
    shapes = [(257,), (2_200_000,), (64, 33), (1_100_000, 3), (4096,), (1,)]
    tensors = _batch(R, shapes, seed=50 + R)
    with session(R):
        outs = rr.all_reduce_many(tensors, "mean")
        sync()
        for t, per in enumerate(tensors):
            want = oracle.all_reduce_closed_form([host(x) for x in per], "mean")
            for r in range(R):
                assert_bits(host(outs[t][r]), want, f"tensor {t} {shapes[t]} rank {r}")


@pytest.mark.parametrize("R,dtype,op", [(4, "f32", "mean"), (4, "i32", "sum"), (8, "f32", "sum"),
                                         (8, "f32", "max"), (3, "f32", "mean")])
def test_all_reduce_many_own_launches(R, dtype, op):
    """Tensors large enough for launches of their own: whole-tile segments
    (the whole-tile kernel), a ragged one and a misaligned view (the general
    kernel), next to small batched ones.  Every tensor equals the ring-order
    oracle and the single-tensor call."""
    tile = 256 * (2 if R < 8 else 1)  # 64 lanes x 4 elements x unroll
    own = (64 << 20) // (2 * R * 4)   # elements per rank for a launch of its own
    whole = -(-own // (R * tile)) * R * tile
    shapes = [(whole,), (whole,), (2 * whole,), (whole + 3,), (whole,), (257,), (whole // R, R)]
    tensors = _batch(R, shapes, seed=70 + R, dtype=dtype)
    # tensor 4: views one element into larger buffers (not on a 256-byte boundary)
    big = gen(R, whole + 1, dtype, "normal", seed=90 + R)
    tensors[4] = [b[1:] for b in big]
    with session(R):
        outs = rr.all_reduce_many(tensors, op)
        sync()
        for t, per in enumerate(tensors):
            hx = [host(x) for x in per]
            want = oracle.all_reduce(hx, op)
            single = rr.all_reduce(per, op)
            sync()
            for r in range(R):
                assert_bits(host(outs[t][r]), want[r], f"tensor {t} {shapes[t]} rank {r}")
                assert_bits(host(single[r]), host(outs[t][r]), f"batched == single, tensor {t}")


def test_occupancy_tuning_keeps_bits():
    """Launches large enough for the occupancy tuner try several wave counts
    while it measures; every call's result equals the oracle's bits, before,
    during and after the choice, for the direct and the ring algorithm."""
    R, N = 8, 4 * 2**20  # 2*R*N*4 = 256 MiB per all-reduce: tuned
    xs = gen(R, N, "f32", "normal", seed=31)
    want = oracle.all_reduce([host(x) for x in xs], "sum")
    for algo in ("auto", "ring"):
        with session(R, algo=algo):
            for call in range(3 * 3 * 2 + 4):
                outs = rr.all_reduce(xs, "sum")
                sync()  # lets the next call read the timers
                for r in (0, call % R):
                    assert_bits(host(outs[r]), want[r], f"{algo} call {call} rank {r}")


def test_all_reduce_many_misaligned_and_repeated():
    """Tensors carved out of one buffer at odd offsets, and several batched
    calls in a row (the descriptor arena alternates and grows)."""
    R = 4
    sizes = [3, 257, 4099, 1, 65_537, 10]
    with session(R):
        for call in range(5):
            bases = gen(R, sum(sizes) + 16 * len(sizes), "f32", "normal", seed=100 + call)
            tensors = []
            for t, n in enumerate(sizes):
                off = sum(sizes[:t]) + 16 * t + (t + call) % 4
                per = []
                for r in range(R):
                    o = off + (r if t % 2 else 0)  # odd tensors: offsets differ per rank
                    per.append(bases[r][o:o + n])
                tensors.append(per)
            grow = sizes * (call + 1)
            tensors = tensors + _batch(R, [(n,) for n in grow], seed=200 + call)
            outs = rr.all_reduce_many(tensors, "mean")
            sync()
            for t, per in enumerate(tensors):
                want = oracle.all_reduce_closed_form([host(x) for x in per], "mean")
                for r in range(R):
                    assert_bits(host(outs[t][r]), want, f"call {call} tensor {t} rank {r}")


# ---------------------------------------------------------------- lifecycle on the GPU

def test_lifecycle_on_gpu():
    xs = gen(2, 100, "f32", "normal", seed=1)
    with pytest.raises(rr.CollectiveError) as e:
        rr.all_reduce(xs, "sum")
    assert e.value.code == rr.RC_ERR_NOT_REGISTERED
    rr.register(2)
    with pytest.raises(rr.CollectiveError) as e:
        rr.register(2)
    assert e.value.code == rr.RC_ERR_DUPLICATE_REGISTRATION
    outs = rr.all_reduce(xs, "sum")
    rr.finish()
    assert_bits(host(outs[0]), oracle.all_reduce_closed_form([host(x) for x in xs], "sum"), "after finish")
    rr.register(2)
    rr.all_reduce_many([xs], "mean")
    assert rr.reset() == rr.RC_OK
    assert rr.reset() == rr.RC_OK
    rr.register(2)
    rr.finish()


@pytest.mark.parametrize("shape", [(), (0,), (2, 3, 4), (1, 2, 1, 3, 1, 2, 1, 5), (3, 0, 7)])
def test_shapes_are_flattened(shape):
    """Scalars, empty shapes, and up to 8 dimensions: every collective works on
    the flattened elements in row-major order, so the bits equal those of the
    same data as 1-D tensors."""
    R = 3
    n = int(np.prod(shape)) if shape else 1
    xs = [si.torch_tensor_for(11, 0, R, r, shape, device=DEV) for r in range(R)]
    hx = [host(x) for x in xs]
    with session(R):
        ar = rr.all_reduce(xs, "sum")
        ag = rr.all_gather(xs)
        red = rr.reduce(xs, 2, "mean")
        torch.cuda.synchronize()
    want = oracle.all_reduce_closed_form([h.reshape(-1) for h in hx], "sum").reshape(shape)
    for r in range(R):
        assert ar[r].shape == torch.Size(shape)
        assert_bits(host(ar[r]), want, f"{shape} all_reduce rank {r}")
        assert_bits(host(ag[r]), np.concatenate([h.reshape(-1) for h in hx]), f"{shape} all_gather rank {r}")
    assert_bits(host(red[2]), oracle.reduce([h.reshape(-1) for h in hx], 2, "mean")[2], f"{shape} reduce")
    if n % R == 0:
        with session(R):
            rs = rr.reduce_scatter(xs, "max")
            torch.cuda.synchronize()
        want_rs = oracle.reduce_scatter([h.reshape(-1) for h in hx], "max")
        for r in range(R):
            assert_bits(host(rs[r]), want_rs[r], f"{shape} reduce_scatter rank {r}")


# ---------------------------------------------------------------- split folds

@pytest.mark.parametrize("case", ["r8_f32_plus8", "r4_i32_plus12", "reduce_r4_plus20", "rs_r8_shards_plus3",
                                  "r8_in_place", "r8_outputs_off_bursts", "r8_ring", "r8_128MiB_plus8",
                                  "r4_64MiB_plus4", "r4_under_64MiB"])
def test_split_folds(case):
    """Folds of 64 MiB and more whose jobs are not whole tiles (segment
    lengths off the 256-byte grid, so each job has its own head and lead)
    run split, in one launch: per job, the first workgroups do the head,
    lead and tail on the general path and the rest the whole tiles of its
    aligned interior on the table kernels (shifted when outputs are off
    their bursts).  Bits against the oracle at those sizes, at the smallest
    split size and just below it (the general kernel), in place too, and
    through the ring's first phase."""
    algo = "ring" if case == "r8_ring" else "direct"
    if case == "r8_128MiB_plus8":
        R, N, dtype, ops = 8, 2**21 + 8, "f32", ("sum", "mean")
    elif case == "r4_64MiB_plus4":
        R, N, dtype, ops = 4, 2**21 + 4, "f32", ("sum", "max")
    elif case == "r4_under_64MiB":
        R, N, dtype, ops = 4, 2**21 - 4, "f32", ("sum", "mean")
    elif case.startswith("r4_i32"):
        R, N, dtype, ops = 4, 2**24 + 12, "i32", ("sum", "max")
    elif case.startswith("reduce"):
        R, N, dtype, ops = 4, 2**24 + 20, "f32", ("sum",)
    elif case.startswith("rs_"):
        R, N, dtype, ops = 8, 8 * (2**21 + 3), "f32", ("sum", "mean")
    else:
        R, N, dtype, ops = 8, 2**24 + 8, "f32", ("sum", "mean")
    dist = "int" if dtype == "i32" else "normal"
    xs = gen(R, N, dtype, dist, seed=6000 + len(case))
    hx = [host(x).copy() for x in xs]
    with session(R, algo=algo):
        for op in ops:
            want = oracle.all_reduce_closed_form(hx, op)
            if case.startswith("reduce"):
                outs = [sentinel_like(torch, x) for x in xs]
                rr.reduce(xs, 2, op, out=[o if r == 2 else None for r, o in enumerate(outs)])
                sync()
                assert_bits(host(outs[2]), want, f"{case} {op} root")
                for r in (0, 1, 3):
                    assert np.all(host(outs[r]).view(np.uint32) == SENTINEL), f"{case}: non-root {r} written"
            elif case.startswith("rs_"):
                M = N // R
                shards = rr.reduce_scatter(xs, op)
                sync()
                for r in range(R):
                    assert_bits(host(shards[r]), want[r * M:(r + 1) * M], f"{case} {op} shard {r}")
            elif case == "r8_in_place":
                ys = [x.clone() for x in xs]
                rr.all_reduce(ys, op, out=ys)
                sync()
                for r in (0, 3, R - 1):
                    assert_bits(host(ys[r]), want, f"{case} {op} rank {r}")
                del ys
            elif case == "r8_outputs_off_bursts":
                offs = [(5 * r) % 16 for r in range(R)]
                bases = [sentinel_like(torch, torch.empty(N + 32, device=DEV)) for _ in range(R)]
                outs = [b[o:o + N] for b, o in zip(bases, offs)]
                rr.all_reduce(xs, op, out=outs)
                sync()
                for r, (b, o) in enumerate(zip(bases, offs)):
                    hb = host(b)
                    assert_bits(hb[o:o + N], want, f"{case} {op} rank {r}")
                    assert np.all(hb.view(np.uint32)[:o] == SENTINEL) and \
                        np.all(hb.view(np.uint32)[o + N:] == SENTINEL), f"{case}: rank {r} written outside"
                del bases, outs
            else:
                outs = rr.all_reduce(xs, op)
                sync()
                for r in range(R):
                    assert_bits(host(outs[r]), want, f"{case} {op} rank {r}")
                del outs
    check_unchanged(xs, hx, case)
