"""The CPU oracle against facts fixed outside of it (see pins.py)."""

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


def _scalar_fold(values, c, R, op):
    """Brute force on one element with numpy float32 scalars, in the ring order
    segment c ends at its owner: (c+1), ..., c."""
    acc = np.float32(values[(c + 1) % R])
    for k in range(2, R + 1):
        v = np.float32(values[(c + k) % R])
        acc = np.float32(acc + v) if op != "max" else np.float32(max(acc, v))
    if op == "mean":
        acc = np.float32(acc / np.float32(R))
    return acc


@pytest.mark.parametrize("R", range(1, 9))
def test_bruteforce_tiny(R):
    """Ring simulation == closed form == scalar loop, bit for bit, on tiny inputs
    (both functions of the oracle are used in the GPU checks)."""
    rng = np.random.default_rng(100 + R)
    for N in (0, 1, 2, 3, 4, 5, 7, 8, 64, 257):
        xs = [(rng.standard_normal(N) * np.exp2(rng.integers(-12, 12, size=N))).astype(np.float32)
              for _ in range(R)]
        S = -(-N // R)
        for op in ("sum", "mean", "max"):
            ring = oracle.all_reduce(xs, op)
            closed = oracle.all_reduce_closed_form(xs, op)
            for r in range(R):
                pins.assert_bits_equal(ring[r], closed, f"ring vs closed R={R} N={N} {op}")
            for i in range(N):
                want = _scalar_fold([x[i] for x in xs], i // S, R, op)
                assert closed[i].view(np.uint32) == np.float32(want).view(np.uint32), (R, N, op, i)


def test_inputs_not_modified_by_any_call():
    rng = np.random.default_rng(7)
    xs = [rng.standard_normal(40).astype(np.float32) for _ in range(4)]
    keep = [x.copy() for x in xs]
    oracle.all_reduce(xs, "sum")
    oracle.reduce(xs, 1, "mean")
    oracle.reduce_scatter(xs, "max")
    oracle.all_gather(xs)
    oracle.broadcast([None, xs[1], None, None])
    oracle.all_reduce_closed_form(xs, "sum")
    oracle.all_reduce_at_many(np.stack(xs), np.arange(40), 40, "sum")
    for x, k in zip(xs, keep):
        assert np.array_equal(x.view(np.uint32), k.view(np.uint32))


def test_errors():
    with pytest.raises(ValueError):
        oracle.reduce_scatter([np.zeros(5, np.float32)] * 2, "sum")
    with pytest.raises(ValueError):
        oracle.all_reduce([np.zeros(5, np.float32), np.zeros(4, np.float32)], "sum")
    with pytest.raises(ValueError):
        oracle.all_reduce([np.zeros(5, np.float32), np.zeros(5, np.int32)], "sum")
    with pytest.raises(ValueError):
        oracle.reduce([np.zeros(5, np.float32)] * 2, 2, "sum")
    with pytest.raises(ValueError):
        oracle.all_reduce([np.zeros(5, np.float64)] * 2, "sum")
