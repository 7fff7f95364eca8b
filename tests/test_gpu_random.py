"""Randomised differential parity: a fixed, seeded stream of valid calls
through the C ABI against the CPU oracle, bit for bit.

Each case draws a collective, a rank count (1-16), a length (empty, short,
ragged, whole tiles), an element type and op, per-rank view offsets of 0-3
elements on inputs and outputs, an in-place layout where the call allows
one, and a session configuration (direct or ring, tile size, persistent
grids, occupancy cap, cache hint).  None of these may change a bit of the
results.  Outputs are views into sentinel-filled buffers, so a write outside
an output fails the case too.  The same seeds give the same cases on every
run, and a failure names its case."""

import random

import numpy as np
import pytest
import torch

import oracle
import rank_reductions_amd as rr
from gpu_util import SENTINEL, assert_bits, host, session

# large finite values overflow to inf in float32 sums, on both sides alike
pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore:overflow encountered:RuntimeWarning")]
DEV = "cuda"

CHUNKS = 16
CASES_PER_CHUNK = 60
RANKS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16]
COLLS = ["all_reduce", "reduce", "broadcast", "reduce_scatter", "all_gather", "all_gather_list",
         "all_to_all_single", "send_recv", "all_reduce_many", "all_reduce_params"]


def draw_len(rng, R, multiple=1):
    """A length: empty, around R, around 256-element tiles, whole tiles per
    segment, or anything up to ~70k; a multiple of `multiple` when asked."""
    kind = rng.randrange(6)
    if kind == 0:
        n = rng.choice([0, 1, 2, 3, 5])
    elif kind == 1:
        n = max(0, R + rng.randint(-2, 2))
    elif kind == 2:
        n = 256 * rng.randint(1, 4) + rng.randint(-3, 3)
    elif kind == 3:
        n = R * 1024 * rng.randint(1, 3)  # whole tiles of every unroll per segment
    else:
        n = rng.randint(0, 70_000)
    n = max(n, 0)
    return n - n % multiple


def values(gen_, n, dtype, op, special):
    """n values on the GPU: ints in [-2^20, 2^20], or float32 N(0,1) with, when
    `special`, signed zeros, subnormals and large finite values mixed in (and
    NaN for Max, whose result for NaN is canonical)."""
    if dtype == "i32":
        return torch.randint(-2 ** 20, 2 ** 20 + 1, (n,), dtype=torch.int32, device=DEV, generator=gen_)
    x = torch.randn(n, device=DEV, generator=gen_)
    if special and n:
        pool = [0.0, -0.0, 1e-40, -1e-40, 2.0 ** -149, 3.0e38]
        if op == "max":
            pool.append(float("nan"))
        idx = torch.randint(0, n, (max(1, n // 8),), device=DEV, generator=gen_)
        pick = torch.randint(0, len(pool), idx.shape, device=DEV, generator=gen_)
        x[idx] = torch.tensor(pool, dtype=torch.float32, device=DEV)[pick]
    return x


class Views:
    """Per-rank views of `n` elements at `off` elements into buffers with 4
    spare elements each side filled with the sentinel, so that writes
    outside a view can be seen."""

    def __init__(self, n, dtype, offs):
        self.n, self.offs = n, offs
        tdt = torch.int32 if dtype == "i32" else torch.float32
        self.bases = [torch.full((n + 8,), SENTINEL, dtype=torch.int32, device=DEV).view(tdt) for _ in offs]
        self.views = [b[o:o + n] for b, o in zip(self.bases, offs)]

    def untouched_outside(self, what):
        for r, (b, o) in enumerate(zip(self.bases, self.offs)):
            hb = host(b).view(np.uint32)
            assert np.all(hb[:o] == SENTINEL) and np.all(hb[o + self.n:] == SENTINEL), \
                f"{what}: rank {r} written outside its output"


def inputs(gen_, R, n, dtype, op, offs, special):
    v = Views(n, dtype, offs)
    for x in v.views:
        x.copy_(values(gen_, n, dtype, op, special))
    return v


def offsets(rng, R):
    mode = rng.randrange(3)
    if mode == 0:
        return [0] * R
    if mode == 1:
        o = rng.randint(1, 3)
        return [o] * R
    return [rng.randint(0, 3) for _ in range(R)]


def fold_op(rng, dtype):
    return rng.choice(["sum", "max"] if dtype == "i32" else ["sum", "mean", "max"])


def run_case(rng, i):
    coll = rng.choice(COLLS)
    R = rng.choice(RANKS)
    if coll == "send_recv" and R == 1:
        R = 2
    dtype = rng.choice(["f32", "f32", "i32"])
    op = fold_op(rng, dtype)
    special = dtype == "f32" and rng.random() < 0.3
    cfg = {"algo": rng.choice(["direct", "ring"]),
           "tile_elems": rng.choice([0, 0, 0, 256, 1024, 4096]),
           "max_workgroups": rng.choice([0, 0, 0, 0, 1, 7, 300]),
           "waves_per_cu": rng.choice([0, 0, 0, 2, 5, 9, 32]),
           "cache_hint": rng.choice(["auto", "auto", "streaming", "normal"])}
    in_place = rng.random() < 0.25
    seed = 1_000 * i + 7
    g = torch.Generator(device=DEV).manual_seed(seed)
    what = f"case {i}: {coll} R={R} {dtype} {op} cfg={cfg} in_place={in_place} special={special} seed={seed}"

    with session(R, **cfg):
        if coll in ("all_reduce", "reduce", "broadcast"):
            n = draw_len(rng, R)
            xin = inputs(g, R, n, dtype, op, offsets(rng, R), special)
            hx = [host(x).copy() for x in xin.views]
            out = Views(n, dtype, offsets(rng, R))
            what += f" n={n} in_offs={xin.offs} out_offs={out.offs}"
            if coll == "all_reduce":
                dst = xin.views if in_place else out.views
                rr.all_reduce(xin.views, op, out=dst)
                torch.cuda.synchronize()
                want = oracle.all_reduce(hx, op)
                for r in range(R):
                    assert_bits(host(dst[r]), want[r], f"{what}: rank {r}")
            elif coll == "reduce":
                root = rng.randrange(R)
                dst = [None] * R
                dst[root] = xin.views[root] if in_place else out.views[root]
                rr.reduce(xin.views, root, op, out=dst)
                torch.cuda.synchronize()
                assert_bits(host(dst[root]), oracle.reduce(hx, root, op)[root], f"{what}: root {root}")
                for r in range(R):  # non-roots' outputs were never handed over: all sentinel
                    if r != root or in_place:
                        assert np.all(host(out.bases[r]).view(np.uint32) == SENTINEL), f"{what}: rank {r} written"
            else:
                src = rng.randrange(R)
                sends = [xin.views[r] if r == src else None for r in range(R)]
                dst = [out.views[r] if r != src else (xin.views[r] if in_place else out.views[r]) for r in range(R)]
                rr.broadcast(sends, out=dst)
                torch.cuda.synchronize()
                want = oracle.broadcast([hx[r] if r == src else None for r in range(R)])
                for r in range(R):
                    assert_bits(host(dst[r]), want[r], f"{what}: rank {r}")
            if not in_place or coll == "broadcast":
                out.untouched_outside(what)
            if not in_place:
                for r in range(R):
                    assert_bits(host(xin.views[r]), hx[r], f"{what}: input {r} changed")
                xin.untouched_outside(what + " (inputs)")
        elif coll in ("reduce_scatter", "all_to_all_single"):
            n = draw_len(rng, R, multiple=R)
            xin = inputs(g, R, n, dtype, op, offsets(rng, R), special)
            hx = [host(x).copy() for x in xin.views]
            if coll == "reduce_scatter":
                m = n // R
                out = Views(m, dtype, offsets(rng, R))
                dst = [xin.views[r][r * m:(r + 1) * m] for r in range(R)] if in_place else out.views
                what += f" n={n} in_offs={xin.offs} out_offs={out.offs}"
                rr.reduce_scatter(xin.views, op, out=dst)
                torch.cuda.synchronize()
                want = oracle.reduce_scatter(hx, op)
            else:
                out = Views(n, dtype, offsets(rng, R))
                dst = out.views
                in_place = False  # no in-place layout exists
                what += f" n={n} in_offs={xin.offs} out_offs={out.offs}"
                rr.all_to_all_single(xin.views, out=dst)
                torch.cuda.synchronize()
                want = oracle.all_to_all_single(hx)
            for r in range(R):
                assert_bits(host(dst[r]), want[r], f"{what}: rank {r}")
            if not in_place:
                out.untouched_outside(what)
                for r in range(R):
                    assert_bits(host(xin.views[r]), hx[r], f"{what}: input {r} changed")
        elif coll in ("all_gather", "all_gather_list"):
            m = draw_len(rng, R) // max(1, R // 4)
            shards = inputs(g, R, m, dtype, op, offsets(rng, R), special)
            hs = [host(x).copy() for x in shards.views]
            if coll == "all_gather":
                out = Views(R * m, dtype, offsets(rng, R))
                what += f" m={m} shard_offs={shards.offs} out_offs={out.offs}"
                if in_place:  # shard r sits at its place in rank r's output
                    for r in range(R):
                        out.views[r][r * m:(r + 1) * m].copy_(shards.views[r])
                    src = [out.views[r][r * m:(r + 1) * m] for r in range(R)]
                else:
                    src = shards.views
                rr.all_gather(src, out=out.views)
                torch.cuda.synchronize()
                want = oracle.all_gather(hs)
                for r in range(R):
                    assert_bits(host(out.views[r]), want[r], f"{what}: rank {r}")
                out.untouched_outside(what)
            else:
                outs = [Views(m, dtype, offsets(rng, R)) for _ in range(R)]
                what += f" m={m} shard_offs={shards.offs}"
                rr.all_gather_list(shards.views, out=[o.views for o in outs])
                torch.cuda.synchronize()
                want = oracle.all_gather_list(hs)
                for r in range(R):
                    for k in range(R):
                        assert_bits(host(outs[r].views[k]), want[r][k], f"{what}: rank {r} shard {k}")
                    outs[r].untouched_outside(f"{what} rank {r}")
            for r in range(R):
                assert_bits(host(shards.views[r]), hs[r], f"{what}: shard {r} changed")
        elif coll == "send_recv":
            n = draw_len(rng, R)
            src, dst_r = rng.sample(range(R), 2)
            xin = inputs(g, 1, n, dtype, op, offsets(rng, 1), special)
            hx = host(xin.views[0]).copy()
            out = Views(n, dtype, offsets(rng, 1))
            what += f" n={n} {src}->{dst_r}"
            rr.send_recv(xin.views[0], src, dst_r, out=out.views[0])
            torch.cuda.synchronize()
            assert_bits(host(out.views[0]), oracle.send_recv(hx), what)
            out.untouched_outside(what)
        elif coll == "all_reduce_many":
            T = rng.randint(1, 6)
            ts = []
            for t in range(T):
                n = draw_len(rng, R)
                ts.append(inputs(g, R, n, dtype, op, offsets(rng, R), special))
            hts = [[host(x).copy() for x in v.views] for v in ts]
            outs = [Views(v.n, dtype, offsets(rng, R)) for v in ts]
            what += f" T={T} ns={[v.n for v in ts]}"
            if rng.random() < 0.5:
                rr.all_reduce_many_static([v.views for v in ts], op, out=[o.views for o in outs])
                what += " static"
            else:
                rr.all_reduce_many([v.views for v in ts], op, out=[o.views for o in outs])
            torch.cuda.synchronize()
            for t in range(T):
                want = oracle.all_reduce(hts[t], op)
                for r in range(R):
                    assert_bits(host(outs[t].views[r]), want[r], f"{what}: tensor {t} rank {r}")
                outs[t].untouched_outside(f"{what} tensor {t}")
        else:  # all_reduce_params, some parameters with accumulators
            ids = rng.sample(range(1, 10_000), rng.randint(1, 5))
            op = "sum" if dtype == "i32" else rng.choice(["sum", "mean"])
            lens = {k: draw_len(rng, R) for k in ids}
            grads = {k: inputs(g, R, lens[k], dtype, op, offsets(rng, R), False) for k in ids}
            with_acc = rng.random() < 0.6
            accs = {k: inputs(g, R, lens[k], dtype, op, offsets(rng, R), False) for k in ids} if with_acc else None
            hg = [{k: host(grads[k].views[r]).copy() for k in ids} for r in range(R)]
            ha = [{k: host(accs[k].views[r]).copy() for k in ids} for r in range(R)] if with_acc else None
            maps = []
            for r in range(R):
                order = ids[:]
                rng.shuffle(order)
                maps.append({k: grads[k].views[r] for k in order})
            amaps = [{k: accs[k].views[r] for k in ids} for r in range(R)] if with_acc else None
            what += f" ids={ids} lens={lens} acc={with_acc}"
            if with_acc and in_place:
                rr.all_reduce_params(maps, op, out=amaps, acc=amaps)
                got = amaps
            else:
                got = rr.all_reduce_params(maps, op, acc=amaps)
            torch.cuda.synchronize()
            want = oracle.all_reduce_params(hg, op, acc=ha)
            for r in range(R):
                for k in ids:
                    assert_bits(host(got[r][k]), want[r][k], f"{what}: rank {r} parameter {k}")


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_calls(chunk):
    rng = random.Random(20_261_203 + chunk)
    for j in range(CASES_PER_CHUNK):
        run_case(rng, chunk * CASES_PER_CHUNK + j)
