"""Helpers shared by the GPU parity tests."""

import contextlib

import numpy as np

import rank_reductions_amd as rr


@contextlib.contextmanager
def session(num_ranks, **cfg):
    rr.register(num_ranks, **cfg)
    try:
        yield
    finally:
        rr.reset()


def host(t):
    return t.detach().cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint32)


def assert_bits(got, want, what=""):
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    gb, wb = bits(got), bits(want)
    if not np.array_equal(gb, wb):
        bad = np.flatnonzero(gb != wb)
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} elements differ; first at {i}: "
                             f"got {got[i]!r} (0x{gb[i]:08x}) want {want[i]!r} (0x{wb[i]:08x})")


def assert_within_bound(got, xs, op, what=""):
    """The order-free tolerance |err| <= 4 R 2^-24 sum_r |x_r| per element
    (Mean: divided by R), against the float64 sum."""
    R = len(xs)
    stack = np.stack([np.asarray(x, dtype=np.float64).reshape(-1) for x in xs])
    exact = stack.sum(axis=0)
    bound = 4 * R * 2.0 ** -24 * np.abs(stack).sum(axis=0)
    g = np.asarray(got, dtype=np.float64).reshape(-1)
    if op == "mean":
        exact = exact / R
        bound = bound / R
    assert np.all(np.abs(g - exact) <= bound), f"{what}: outside the tolerance"


SENTINEL = 0x7FC0DEAD  # a NaN payload no collective produces


def sentinel_like(torch, t):
    return torch.full(t.shape, SENTINEL, dtype=torch.int32, device=t.device).view(t.dtype) \
        if t.dtype == torch.float32 else torch.full(t.shape, SENTINEL, dtype=torch.int32, device=t.device)
