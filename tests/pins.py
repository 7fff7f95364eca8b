"""Pins that tie the CPU oracle to facts fixed outside of it.

Each pin takes the oracle module as an argument so the same checks can be run
against deliberately broken copies of the oracle (see the mutation tests).
A pin raises AssertionError (or the oracle's own error) when it fails.

Where each fact comes from:
* hand-derived worked examples of the ring order (tests/golden), following
  the ring AllReduce of the ruCCL README (ja), "CUDA tensor example";
* exact integer arithmetic: float32 inputs that are integers of magnitude at
  most 2^20, summed over at most 8 ranks, have exact float32 sums in any order;
* Higham's bound for recursive summation against an exactly rounded sum;
* library routines for order-free results (numpy integer sum and max,
  concatenation for all-gather);
* invariants the pages state: inputs unchanged, one broadcast sender, only the
  root receiving a reduce, reduce_scatter = reduce then scatter, and the
  gather of the scattered shards equal to the all-reduce.
"""

import math
from pathlib import Path

import numpy as np

U = 2.0 ** -24
GOLDEN = Path(__file__).resolve().parent / "golden"


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if np.asarray(a).dtype == np.float32 else np.int32)


def assert_bits_equal(a, b, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert a.dtype == b.dtype, f"{what}: dtype {a.dtype} != {b.dtype}"
    if not np.array_equal(bits(a), bits(b)):
        bad = np.flatnonzero(bits(a).reshape(-1) != bits(b).reshape(-1))
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} elements differ, first at {i}: "
                             f"{a.reshape(-1)[i]!r} vs {b.reshape(-1)[i]!r}")


def load_order_examples():
    examples = []
    cur = None
    for line in (GOLDEN / "ring_order_examples.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "example":
            cur = {"name": rest[0]}
            examples.append(cur)
        elif key in ("R", "N"):
            cur[key] = int(rest[0])
        else:
            cur[key] = np.array([int(w, 16) for w in rest], dtype=np.uint32).view(np.float32)
    return examples


def _rng(seed):
    return np.random.default_rng(seed)


def _int_valued(rng, R, N):
    return [rng.integers(-(1 << 20), (1 << 20) + 1, size=N).astype(np.float32) for _ in range(R)]


# ---------------------------------------------------------------------------

def pin_segments(orc):
    """The reading S = ceil(N/R), written out for the pages' own size (257 FP32
    elements over 4 ranks) and for empty and ragged cases."""
    assert orc.segment_bounds(257, 4) == [(0, 65), (65, 130), (130, 195), (195, 257)]
    assert orc.segment_bounds(4, 3) == [(0, 2), (2, 4), (4, 4)]
    assert orc.segment_bounds(0, 5) == [(0, 0)] * 5
    assert orc.segment_bounds(3, 8) == [(0, 1), (1, 2), (2, 3)] + [(3, 3)] * 5
    assert orc.segment_bounds(16, 8) == [(2 * c, 2 * c + 2) for c in range(8)]


def pin_worked_examples(orc):
    """Hand-derived ring-order examples (golden file): sum and mean bits."""
    for ex in load_order_examples():
        R, N = ex["R"], ex["N"]
        xs = [np.full(N, ex["values"][r], dtype=np.float32) for r in range(R)]
        for op in (orc.SUM, orc.MEAN):
            want = ex[op]
            outs = orc.all_reduce(xs, op)
            for r in range(R):
                assert_bits_equal(outs[r], want, f"{ex['name']} all_reduce {op} rank {r}")
            assert_bits_equal(orc.all_reduce_closed_form(xs, op), want, f"{ex['name']} closed {op}")
            got = orc.all_reduce_at_many(np.stack(xs), np.arange(N), N, op)
            assert_bits_equal(got, want, f"{ex['name']} at_many {op}")
            for i in range(N):
                assert_bits_equal(np.array([orc.all_reduce_at(np.stack(xs)[:, i], i, N, op)]),
                                  want[i:i + 1], f"{ex['name']} at {i} {op}")
            for root in range(R):
                red = orc.reduce(xs, root, op)
                assert_bits_equal(red[root], want, f"{ex['name']} reduce root {root} {op}")
            if N % R == 0:
                m = N // R
                shards = orc.reduce_scatter(xs, op)
                for r in range(R):
                    assert_bits_equal(shards[r], want[r * m:(r + 1) * m], f"{ex['name']} rs {op} {r}")
            many = orc.all_reduce_many([xs, xs], op)
            for t in range(2):
                for r in range(R):
                    assert_bits_equal(many[t][r], want, f"{ex['name']} many {op}")


def pin_integer_exact(orc):
    """Integer-valued float32 inputs (|x| <= 2^20, R <= 8) have exact sums in
    any order, so every result must equal the int64 sum.  Mean must equal the
    float64 quotient rounded once to float32 (double rounding is harmless for
    division when 53 >= 2*24 + 2)."""
    rng = _rng(11)
    for R in range(1, 9):
        for N in (0, 1, 5, 64, 257, 1000):
            xs = _int_valued(rng, R, N)
            exact = np.sum(np.stack(xs).astype(np.int64), axis=0) if N else np.zeros(0, np.int64)
            want_sum = exact.astype(np.float32)
            want_mean = (exact.astype(np.float64) / R).astype(np.float32)
            for op, want in ((orc.SUM, want_sum), (orc.MEAN, want_mean)):
                outs = orc.all_reduce(xs, op)
                for r in range(R):
                    assert_bits_equal(outs[r], want, f"R={R} N={N} all_reduce {op} rank {r}")
                assert_bits_equal(orc.all_reduce_closed_form(xs, op), want, f"closed {op}")
                if N:
                    idx = np.arange(N)
                    assert_bits_equal(orc.all_reduce_at_many(np.stack(xs), idx, N, op), want, "at_many")
                    i = N - 1
                    assert_bits_equal(np.array([orc.all_reduce_at(np.stack(xs)[:, i], i, N, op)]),
                                      want[i:i + 1], "at last")
                root = (R - 1) // 2
                red = orc.reduce(xs, root, op)
                assert_bits_equal(red[root], want, f"reduce {op}")
                assert all(red[r] is None for r in range(R) if r != root)
                if N % R == 0:
                    m = N // R
                    shards = orc.reduce_scatter(xs, op)
                    for r in range(R):
                        assert_bits_equal(shards[r], want[r * m:(r + 1) * m], f"rs {op} rank {r}")
            if N:
                many = orc.all_reduce_many([xs, _int_valued(rng, R, 3)], orc.SUM)
                assert_bits_equal(many[0][R - 1], want_sum, "all_reduce_many tensor 0")


def pin_error_bound(orc):
    """Any fold order of R float32 values lies within (R-1) * 2^-24 * sum|x_r|
    of the exact sum (Higham, recursive summation); Mean within that bound / R
    plus one more rounding of s/R.  The exact sum is math.fsum."""
    rng = _rng(12)
    for R in (2, 3, 5, 8):
        N = 257
        # wide dynamic range so that rounding actually happens
        xs = [(rng.standard_normal(N) * np.exp2(rng.integers(-20, 20, size=N))).astype(np.float32)
              for _ in range(R)]
        stack = np.stack(xs).astype(np.float64)
        exact = np.array([math.fsum(stack[:, i]) for i in range(N)])
        absum = np.abs(stack).sum(axis=0)
        got = orc.all_reduce(xs, orc.SUM)[0].astype(np.float64)
        bound = (R - 1) * U * absum
        assert np.all(np.abs(got - exact) <= bound), "sum outside the recursive-summation bound"
        mean = orc.all_reduce(xs, orc.MEAN)[0].astype(np.float64)
        mbound = bound / R + U * np.abs(exact / R) * (1 + R * U)
        assert np.all(np.abs(mean - exact / R) <= mbound), "mean outside its bound"


def pin_i32(orc):
    """int32 Sum wraps (numpy's int64 sum taken modulo 2^32) and Max is numpy's
    max; both are independent of the order."""
    rng = _rng(13)
    for R in (1, 2, 4, 7, 8):
        for N in (0, 3, 257, 1024):
            xs = [rng.integers(-(1 << 31), 1 << 31, size=N, dtype=np.int64).astype(np.int32)
                  for _ in range(R)]
            stack = np.stack(xs)
            want_sum = (np.sum(stack.astype(np.int64), axis=0) % (1 << 32)).astype(np.uint32).view(np.int32)
            want_max = np.max(stack, axis=0) if N else np.zeros(0, np.int32)
            for op, want in ((orc.SUM, want_sum), (orc.MAX, want_max)):
                outs = orc.all_reduce(xs, op)
                for r in range(R):
                    assert_bits_equal(outs[r], want, f"i32 R={R} N={N} {op}")
                assert_bits_equal(orc.all_reduce_closed_form(xs, op), want, f"i32 closed {op}")
                red = orc.reduce(xs, R - 1, op)
                assert_bits_equal(red[R - 1], want, f"i32 reduce {op}")
                if N:
                    assert_bits_equal(orc.all_reduce_at_many(stack, np.arange(N), N, op), want, "i32 at")
                if N % R == 0:
                    m = N // R
                    shards = orc.reduce_scatter(xs, op)
                    for r in range(R):
                        assert_bits_equal(shards[r], want[r * m:(r + 1) * m], f"i32 rs {op}")
    try:
        orc.all_reduce([np.zeros(4, np.int32)] * 2, orc.MEAN)
    except ValueError:
        pass
    else:
        raise AssertionError("int32 Mean must be rejected")


def pin_f32_max(orc):
    """float32 Max: numpy's max on ordinary values; a NaN anywhere gives the
    canonical quiet NaN; +0 wins over -0 unless every operand is -0."""
    rng = _rng(14)
    for R in (1, 2, 3, 8):
        N = 301
        xs = [rng.standard_normal(N).astype(np.float32) for _ in range(R)]
        stack = np.stack(xs)
        want = np.max(stack, axis=0)
        assert_bits_equal(orc.all_reduce(xs, orc.MAX)[R // 2], want, f"max R={R}")
        assert_bits_equal(orc.all_reduce_closed_form(xs, orc.MAX), want, "max closed")
        assert_bits_equal(orc.all_reduce_at_many(stack, np.arange(N), N, orc.MAX), want, "max at")
    # NaN and signed zeros
    R = 4
    xs = [np.array([1.0, 0.0, -0.0, -0.0, np.nan, -np.inf], dtype=np.float32) for _ in range(R)]
    xs[2] = np.array([np.nan, -0.0, -0.0, -0.0, 3.0, -np.inf], dtype=np.float32)
    xs[1] = xs[1].copy()
    xs[1].view(np.uint32)[4] = 0xFFC00001  # a NaN with another payload and sign
    want = np.array([0x7FC00000, 0x00000000, 0x80000000, 0x80000000, 0x7FC00000, 0xFF800000],
                    dtype=np.uint32).view(np.float32)
    for r, out in enumerate(orc.all_reduce(xs, orc.MAX)):
        assert_bits_equal(out, want, f"max special rank {r}")
    assert_bits_equal(orc.all_reduce_closed_form(xs, orc.MAX), want, "max special closed")


def pin_mean_power_of_two(orc):
    """For R a power of two, dividing by R is exact scaling, so Mean equals the
    Sum times 2^-k bit for bit (also when the result is subnormal)."""
    rng = _rng(15)
    for R in (1, 2, 4, 8):
        N = 200
        xs = [(rng.standard_normal(N) * 1e-37).astype(np.float32) for _ in range(R)]
        s = orc.all_reduce(xs, orc.SUM)[0]
        m = orc.all_reduce(xs, orc.MEAN)[0]
        assert_bits_equal(m, np.ldexp(s, -int(math.log2(R))).astype(np.float32), f"mean R={R}")


def pin_subnormals(orc):
    """Subnormal inputs are kept (no flush to zero): integer multiples of
    2^-149 add exactly while the sum stays below 2^24 such units."""
    rng = _rng(16)
    tiny = np.float32(2.0 ** -149)
    for R in (2, 4, 8):
        N = 100
        ks = [rng.integers(-1000, 1001, size=N) for _ in range(R)]
        xs = [(k.astype(np.float32) * tiny).astype(np.float32) for k in ks]
        exact = np.sum(np.stack(ks), axis=0)
        want = (exact.astype(np.float32) * tiny).astype(np.float32)
        assert_bits_equal(orc.all_reduce(xs, orc.SUM)[0], want, f"subnormal R={R}")


def pin_broadcast(orc):
    """One sender; every rank receives the sender's bytes; zero or two senders
    is an error (ruCCL README, sections 2 and 4)."""
    rng = _rng(17)
    for R in range(1, 9):
        for dtype in (np.float32, np.int32):
            src = rng.integers(-(1 << 31), 1 << 31, size=257, dtype=np.int64).astype(np.int32)
            src = src.view(dtype)
            for sender in {0, R - 1, R // 2}:
                sends = [None] * R
                sends[sender] = src
                keep = src.copy()
                outs = orc.broadcast(sends)
                assert len(outs) == R
                for r in range(R):
                    assert np.array_equal(outs[r].view(np.uint8), keep.view(np.uint8)), "broadcast bytes"
                assert np.array_equal(src.view(np.uint8), keep.view(np.uint8)), "sender changed"
    for bad in ([None, None, None], [np.zeros(3, np.float32)] * 2):
        try:
            orc.broadcast(bad)
        except ValueError:
            continue
        raise AssertionError("sender count != 1 must be rejected")


def pin_all_gather(orc):
    """all_gather_into_tensor: every rank's output is the concatenation of the
    shards in rank order (numpy.concatenate)."""
    rng = _rng(18)
    for R in range(1, 9):
        for M in (0, 1, 7, 64):
            shards = [rng.integers(-(1 << 31), 1 << 31, size=M, dtype=np.int64).astype(np.int32).view(np.float32)
                      for _ in range(R)]
            want = np.concatenate(shards) if M else np.zeros(0, np.float32)
            outs = orc.all_gather(shards)
            for r in range(R):
                assert_bits_equal(outs[r], want, f"all_gather R={R} M={M} rank {r}")


def pin_invariants(orc):
    """Invariants the pages fix: inputs unchanged (ruCCL example), all ranks
    identical, reduce's root equal to all_reduce with other ranks receiving
    nothing, gather of the scattered shards equal to the all-reduce, and a
    single rank as the identity."""
    rng = _rng(19)
    for R in range(1, 9):
        for N in (0, 1, 8, 257, 512):
            xs = [rng.standard_normal(N).astype(np.float32) for _ in range(R)]
            keep = [x.copy() for x in xs]
            for op in (orc.SUM, orc.MEAN, orc.MAX):
                ar = orc.all_reduce(xs, op)
                for r in range(R):
                    assert_bits_equal(ar[r], ar[0], "ranks differ")
                for root in range(R):
                    red = orc.reduce(xs, root, op)
                    assert_bits_equal(red[root], ar[0], "reduce != all_reduce")
                    assert all(red[r] is None for r in range(R) if r != root), "non-root received"
                if N % R == 0:
                    gathered = orc.all_gather(orc.reduce_scatter(xs, op))
                    for r in range(R):
                        assert_bits_equal(gathered[r], ar[0], "AG(RS(x)) != AR(x)")
                if R == 1:
                    assert_bits_equal(ar[0], xs[0], "single rank is the identity")
            for r in range(R):
                assert_bits_equal(xs[r], keep[r], "input modified")


def load_all_to_all_example():
    ex = {"in": {}, "out": {}}
    for line in (GOLDEN / "all_to_all_example.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "R":
            ex["R"] = int(rest[0])
        else:
            ex[key][int(rest[0])] = np.array([int(v) for v in rest[1:]], dtype=np.int32)
    return ex


def pin_all_to_all(orc):
    """all_to_all_single (Communicator page): the hand-derived worked example
    in tests/golden; applying it twice gives back the inputs (chunk d of rank
    s goes to chunk s of rank d, and back); every element keeps its bits
    (a permutation: the multiset of all ranks' values is unchanged); R = 1 is
    a copy; a length not divisible by R is refused."""
    ex = load_all_to_all_example()
    R = ex["R"]
    got = orc.all_to_all_single([ex["in"][r] for r in range(R)])
    for r in range(R):
        assert_bits_equal(got[r], ex["out"][r], f"worked example rank {r}")
    rng = _rng(37)
    for R in (1, 2, 3, 5, 8):
        for m in (0, 1, 3, 64):
            xs = [rng.standard_normal((R * m,)).astype(np.float32) for _ in range(R)]
            once = orc.all_to_all_single(xs)
            twice = orc.all_to_all_single(once)
            for r in range(R):
                assert_bits_equal(twice[r], xs[r], f"R={R} m={m}: twice is not the identity")
            a = np.sort(np.concatenate([bits(x).reshape(-1) for x in xs]))
            b = np.sort(np.concatenate([bits(x).reshape(-1) for x in once]))
            assert np.array_equal(a, b), "values changed"
            if R == 1:
                assert_bits_equal(once[0], xs[0], "single rank is a copy")
    try:
        orc.all_to_all_single([np.zeros(5, np.float32)] * 2)
    except orc.OracleError:
        pass
    else:
        raise AssertionError("a length not divisible by R was accepted")


def pin_all_gather_list(orc):
    """The list form of all_gather (Communicator.all_gather) holds, rank by
    rank, the pieces of the single-tensor form (all_gather_into_tensor, pinned
    to numpy.concatenate): output k of every rank is rank k's input, bit for
    bit, as a copy; shapes are kept."""
    rng = _rng(41)
    for R in (1, 2, 4, 7):
        shards = [rng.standard_normal((3, 5)).astype(np.float32) for _ in range(R)]
        out = orc.all_gather_list(shards)
        flat = np.concatenate([s.reshape(-1) for s in shards])
        assert len(out) == R
        for r in range(R):
            assert len(out[r]) == R
            assert_bits_equal(np.concatenate([o.reshape(-1) for o in out[r]]), flat, f"R={R} rank {r}")
            for k in range(R):
                assert out[r][k].shape == (3, 5)
                assert not np.shares_memory(out[r][k], shards[k]), "output aliases an input"
    x = np.arange(7, dtype=np.int32)
    y = orc.send_recv(x)
    assert_bits_equal(y, x, "send/recv copies")
    assert not np.shares_memory(x, y)


def _param_maps(rng, R, specs, int_valued=True, seed_order=0):
    """R maps {id: array}; rank r inserts its entries in its own order."""
    order_rng = _rng(1000 + seed_order)
    maps = []
    for r in range(R):
        entries = {}
        for pid, shape in specs:
            n = int(np.prod(shape)) if shape else 1
            if int_valued:
                v = rng.integers(-(1 << 20), (1 << 20) + 1, size=n).astype(np.float32)
            else:
                v = rng.standard_normal(n).astype(np.float32)
            entries[pid] = v.reshape(shape)
        keys = list(entries)
        order_rng.shuffle(keys)
        maps.append({k: entries[k] for k in keys})
    return maps


PARAM_SPECS = [(7, (3, 5)), (3, (257,)), (11, (0,)), (0, ()), (42, (64,)), (5, (2, 2, 3))]


def pin_params(orc):
    """Whole-gradient sync keyed by parameter ID (ruCCL README section 6):
    entries pair by ID whatever order each rank lists them in, every
    parameter gets the exact reduction of its own R tensors (integer-valued
    float32 sums are exact in any order, so they must equal numpy's int64
    sum; Mean is that sum divided by R and rounded once), all ranks agree,
    inputs are unchanged, and ID, dtype and shape disagreements are reported
    as such (IDs first, then dtype before shape)."""
    rng = _rng(23)
    for R in (1, 2, 3, 5, 8):
        maps = _param_maps(rng, R, PARAM_SPECS, seed_order=R)
        keep = [{k: v.copy() for k, v in m.items()} for m in maps]
        for op in (orc.SUM, orc.MEAN):
            out = orc.all_reduce_params(maps, op)
            assert len(out) == R
            for pid, shape in PARAM_SPECS:
                exact = np.sum(np.stack([maps[r][pid].astype(np.int64) for r in range(R)]), axis=0)
                want = exact.astype(np.float32) if op == orc.SUM else \
                    (exact.astype(np.float64) / R).astype(np.float32)
                for r in range(R):
                    assert set(out[r]) == {p for p, _ in PARAM_SPECS}, "ID set changed"
                    assert_bits_equal(out[r][pid], want.reshape(shape), f"R={R} {op} id {pid} rank {r}")
        for r in range(R):
            for pid in keep[r]:
                assert_bits_equal(maps[r][pid], keep[r][pid], "input modified")

    def expect(kind, maps):
        try:
            orc.all_reduce_params(maps, orc.MEAN)
        except orc.ParamMismatch as e:
            assert e.kind == kind, f"reported {e.kind!r}, expected {kind!r}"
            return
        raise AssertionError(f"{kind} mismatch not reported")

    base = _param_maps(rng, 3, PARAM_SPECS, seed_order=99)
    missing = [dict(m) for m in base]
    del missing[2][42]
    expect("ids", missing)
    extra = [dict(m) for m in base]
    extra[1][99] = np.zeros(4, np.float32)
    expect("ids", extra)
    renamed = [dict(m) for m in base]
    renamed[0][43] = renamed[0].pop(42)
    expect("ids", renamed)
    shape = [dict(m) for m in base]
    shape[1][7] = shape[1][7].reshape(5, 3)
    expect("shape", shape)
    dtype = [dict(m) for m in base]
    dtype[2][3] = dtype[2][3].astype(np.int32)
    expect("dtype", dtype)
    both = [dict(m) for m in base]
    both[2][5] = np.zeros((12,), np.int32)
    expect("dtype", both)


def pin_params_accumulated(orc):
    """The sync of accumulated gradients (ruCCL README section 6 with the
    GradientsAccumulator of RUDA "Training and state saving"): integer-valued
    accumulators and gradients reduce to the exact int64 sum of acc + grad
    over ranks (Mean: divided by R, rounded once); parameters without
    accumulators keep the plain result; an accumulator on some ranks only, or
    with Max, is refused."""
    rng = _rng(31)
    R = 4
    grads = _param_maps(rng, R, PARAM_SPECS, seed_order=7)
    accs = [{pid: rng.integers(-(1 << 20), (1 << 20) + 1, size=np.shape(m[pid])).astype(np.float32)
             for pid in (7, 3, 42)} for m in grads]
    for op in (orc.SUM, orc.MEAN):
        out = orc.all_reduce_params(grads, op, acc=accs)
        for pid, shape in PARAM_SPECS:
            terms = [grads[r][pid].astype(np.int64) + (accs[r][pid].astype(np.int64) if pid in accs[r] else 0)
                     for r in range(R)]
            exact = np.sum(np.stack(terms), axis=0)
            want = exact.astype(np.float32) if op == orc.SUM else (exact.astype(np.float64) / R).astype(np.float32)
            for r in range(R):
                assert_bits_equal(out[r][pid], want.reshape(shape), f"{op} id {pid} rank {r} with accumulators")
    partial = [dict(a) for a in accs]
    del partial[2][3]
    for bad, op in ((partial, orc.MEAN), (accs, orc.MAX)):
        try:
            orc.all_reduce_params(grads, op, acc=bad)
        except orc.OracleError:
            continue
        raise AssertionError("an invalid accumulator set was accepted")


def pin_accumulate(orc):
    """GradientsAccumulator.accumulate (RUDA "Training and state saving"):
    adds without averaging, so integer-valued float32 gradients accumulate to
    their exact int64 sum; the first gradient is copied, not aliased; int32
    wraps; a shape change is refused."""
    rng = _rng(29)
    grads = [rng.integers(-(1 << 20), (1 << 20) + 1, size=(4, 33)).astype(np.float32) for _ in range(6)]
    acc = None
    for k, g in enumerate(grads):
        acc = orc.accumulate(acc, g)
        exact = np.sum(np.stack([x.astype(np.int64) for x in grads[:k + 1]]), axis=0)
        assert_bits_equal(acc, exact.astype(np.float32), f"after {k + 1} microbatches")
    first = np.ones(5, np.float32)
    acc = orc.accumulate(None, first)
    acc[0] = 7.0
    assert first[0] == 1.0, "the accumulator aliases the caller's gradient"
    top = np.array([2 ** 31 - 1, -2 ** 31], np.int32)
    assert_bits_equal(orc.accumulate(top, np.array([1, -1], np.int32)),
                      np.array([-2 ** 31, 2 ** 31 - 1], np.int32), "int32 wraps")
    try:
        orc.accumulate(np.zeros(4, np.float32), np.zeros(5, np.float32))
    except orc.OracleError:
        pass
    else:
        raise AssertionError("shape change accepted")


ALL_PINS = [
    pin_segments,
    pin_worked_examples,
    pin_integer_exact,
    pin_error_bound,
    pin_i32,
    pin_f32_max,
    pin_mean_power_of_two,
    pin_subnormals,
    pin_broadcast,
    pin_all_gather,
    pin_invariants,
    pin_params,
    pin_params_accumulated,
    pin_accumulate,
    pin_all_to_all,
    pin_all_gather_list,
]
