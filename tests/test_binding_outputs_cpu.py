"""The binding checks every caller-supplied output tensor before calling the
library: the C ABI carries only the input's shape, so an output of the wrong
size or dtype would otherwise be written past its end or misread.

On the CPU the tensors are host tensors: a bad output raises CollectiveError
with the matching status before any pointer is taken, while an output that
passes the checks goes on to the device check of the pointer marshalling
(ValueError: tensors must be on a CUDA device), which shows that the output
checks let it through.
"""

import pytest
import torch

import rank_reductions_amd as rr

SHAPE = rr.RC_ERR_SHAPE_MISMATCH
DTYPE = rr.RC_ERR_DTYPE_MISMATCH
INVAL = rr.RC_ERR_INVALID_ARGUMENT

R, N = 4, 64


def xs(n=N, dtype=torch.float32, R=R):
    return [torch.zeros(n, dtype=dtype) for _ in range(R)]


def code_of(fn):
    with pytest.raises(rr.CollectiveError) as e:
        fn()
    return e.value.code


def passes_checks(fn):
    """The output checks let the call through: it fails only at the host
    tensors' pointers."""
    with pytest.raises(ValueError, match="CUDA"):
        fn()


def test_all_reduce_outputs():
    x = xs()
    assert code_of(lambda: rr.all_reduce(x, out=xs(N - 1))) == SHAPE
    assert code_of(lambda: rr.all_reduce(x, out=xs(dtype=torch.int32))) == DTYPE
    assert code_of(lambda: rr.all_reduce(x, out=xs()[:3])) == INVAL
    assert code_of(lambda: rr.all_reduce(x, out=[torch.zeros(2 * N)[::2] for _ in range(R)])) == INVAL
    assert code_of(lambda: rr.all_reduce(x, out=xs()[:3] + [torch.zeros(N + 1)])) == SHAPE
    passes_checks(lambda: rr.all_reduce(x, out=xs()))
    passes_checks(lambda: rr.all_reduce(x, out=x))  # in place


def test_reduce_root_output():
    x = xs()
    assert code_of(lambda: rr.reduce(x, 2, out=[None, None, torch.zeros(N // 2), None])) == SHAPE
    assert code_of(lambda: rr.reduce(x, 2, out=[None, None, torch.zeros(N, dtype=torch.int32), None])) == DTYPE
    assert code_of(lambda: rr.reduce(x, 2, out=[None, None, None, None])) == INVAL
    passes_checks(lambda: rr.reduce(x, 2, out=[None, None, torch.zeros(N), None]))


def test_broadcast_outputs():
    src = torch.zeros(N)
    sends = [None, src, None, None]
    assert code_of(lambda: rr.broadcast(sends, out=[torch.zeros(N), None, torch.zeros(N - 4), torch.zeros(N)])) == SHAPE
    bad = [torch.zeros(N), None, torch.zeros(N, dtype=torch.int32), torch.zeros(N)]
    assert code_of(lambda: rr.broadcast(sends, out=bad)) == DTYPE
    passes_checks(lambda: rr.broadcast(sends, out=[torch.zeros(N), None, torch.zeros(N), torch.zeros(N)]))


def test_reduce_scatter_outputs():
    x = xs()
    assert code_of(lambda: rr.reduce_scatter(x, out=xs(N))) == SHAPE          # full length, not N/R
    assert code_of(lambda: rr.reduce_scatter(x, out=xs(N // R - 1))) == SHAPE
    assert code_of(lambda: rr.reduce_scatter(x, out=xs(N // R, torch.int32))) == DTYPE
    passes_checks(lambda: rr.reduce_scatter(x, out=xs(N // R)))


def test_all_gather_outputs():
    shards = xs(16)
    assert code_of(lambda: rr.all_gather(shards, out=xs(16))) == SHAPE       # a shard's size, not R*M
    assert code_of(lambda: rr.all_gather(shards, out=xs(R * 16, torch.int32))) == DTYPE
    passes_checks(lambda: rr.all_gather(shards, out=xs(R * 16)))


def test_batched_outputs():
    ts = [xs(N), xs(7)]
    good = [xs(N), xs(7)]
    for fn in (rr.all_reduce_many, rr.all_reduce_many_static):
        assert code_of(lambda: fn(ts, out=[xs(N), xs(6)])) == SHAPE
        assert code_of(lambda: fn(ts, out=[xs(N), xs(7, torch.int32)])) == DTYPE
        assert code_of(lambda: fn(ts, out=[xs(N)])) == INVAL
        passes_checks(lambda: fn(ts, out=good))


def test_list_all_gather_outputs():
    shards = xs(8)
    good = [[torch.zeros(8) for _ in range(R)] for _ in range(R)]
    bad = [[torch.zeros(8) for _ in range(R)] for _ in range(R)]
    bad[3][1] = torch.zeros(7)
    assert code_of(lambda: rr.all_gather_list(shards, out=bad)) == SHAPE
    bad[3][1] = torch.zeros(8, dtype=torch.int32)
    assert code_of(lambda: rr.all_gather_list(shards, out=bad)) == DTYPE
    assert code_of(lambda: rr.all_gather_list(shards, out=good[:2])) == INVAL
    passes_checks(lambda: rr.all_gather_list(shards, out=good))


def test_all_to_all_and_send_recv_outputs():
    x = xs()
    assert code_of(lambda: rr.all_to_all_single(x, out=xs(N // R))) == SHAPE
    passes_checks(lambda: rr.all_to_all_single(x, out=xs()))
    assert code_of(lambda: rr.send_recv(x[0], 0, 1, out=torch.zeros(N - 1))) == SHAPE
    assert code_of(lambda: rr.send_recv(x[0], 0, 1, out=torch.zeros(N, dtype=torch.int32))) == DTYPE
    passes_checks(lambda: rr.send_recv(x[0], 0, 1, out=torch.zeros(N)))


def test_params_outputs_and_accumulators():
    grads = [{7: torch.zeros(N), 3: torch.zeros(5)} for _ in range(R)]
    outs = [{7: torch.zeros(N), 3: torch.zeros(5)} for _ in range(R)]
    bad = [{7: torch.zeros(N), 3: torch.zeros(4)} for _ in range(R)]
    assert code_of(lambda: rr.all_reduce_params(grads, out=bad)) == SHAPE
    assert code_of(lambda: rr.all_reduce_params(grads, out=[{7: torch.zeros(N)} for _ in range(R)])) == INVAL
    accs = [{7: torch.zeros(N, dtype=torch.int32)} for _ in range(R)]
    assert code_of(lambda: rr.all_reduce_params(grads, out=outs, acc=accs)) == DTYPE
    accs = [{3: torch.zeros(6)} for _ in range(R)]
    assert code_of(lambda: rr.all_reduce_params(grads, out=outs, acc=accs)) == SHAPE
    passes_checks(lambda: rr.all_reduce_params(grads, out=outs))


def test_per_rank_outputs():
    x = torch.zeros(N)
    assert code_of(lambda: rr.rank_all_reduce(0, x, out=torch.zeros(N - 1))) == SHAPE
    assert code_of(lambda: rr.rank_reduce(2, x, 2, out=torch.zeros(N, dtype=torch.int32))) == DTYPE
    assert code_of(lambda: rr.rank_reduce_scatter(1, x, R, out=torch.zeros(N))) == SHAPE
    assert code_of(lambda: rr.rank_all_gather(1, x, R, out=torch.zeros(N))) == SHAPE
    assert code_of(lambda: rr.rank_all_gather_list(1, x, R, out=[torch.zeros(N)] * (R - 1))) == INVAL
    assert code_of(lambda: rr.rank_all_gather_list(1, x, R, out=[torch.zeros(N - 1)] * R)) == SHAPE
    assert code_of(lambda: rr.rank_all_to_all_single(1, x, out=torch.zeros(2 * N))) == SHAPE
    grads = {1: x}
    assert code_of(lambda: rr.rank_all_reduce_params(0, grads, out={1: torch.zeros(3)})) == SHAPE
    passes_checks(lambda: rr.rank_all_reduce(0, x, out=torch.zeros(N)))


def test_communicator_methods_check_outputs():
    comm = rr.Communicator._from_endpoint(1, R)  # rank 1 of 4, no session needed for these checks
    x = torch.zeros(N)
    assert code_of(lambda: comm.all_gather_into_tensor(torch.zeros(N), x)) == SHAPE
    assert code_of(lambda: comm.reduce_scatter_tensor(torch.zeros(N), x)) == SHAPE
    assert code_of(lambda: comm.all_gather([torch.zeros(N)] * R, torch.zeros(N, dtype=torch.int32))) == DTYPE
    assert code_of(lambda: comm.all_to_all_single(torch.zeros(N + 4), x)) == SHAPE
