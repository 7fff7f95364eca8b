"""Planted mistakes in the oracle must be caught by the pins.

Each case copies the oracle's source, plants one plausible mistake (a wrong
ring index, a dropped term, a wrong sign, a wrong divisor, transposed shards,
...) and runs every pin on the broken copy: at least one pin must fail.
Everything here runs on the CPU; the real oracle is never modified.
"""

import types
from pathlib import Path

import pytest

import pins

SOURCE = (Path(__file__).resolve().parent.parent / "oracle" / "ring.py").read_text()

MUTATIONS = {
    "rs_sends_wrong_segment": ("c = (r - s - 1) % R", "c = (r - s) % R"),
    "rs_drops_own_term": ("state[dst][lo:hi] = combine(received, flat[dst][lo:hi], op)",
                          "state[dst][lo:hi] = received"),
    "rs_keeps_own_only": ("state[dst][lo:hi] = combine(received, flat[dst][lo:hi], op)",
                          "state[dst][lo:hi] = flat[dst][lo:hi]"),
    "add_is_subtract": ("return np.add(a, b, dtype=np.float32)",
                        "return np.subtract(a, b, dtype=np.float32)"),
    "i32_add_is_subtract": ("wide = a.astype(np.int64) + b.astype(np.int64)",
                            "wide = a.astype(np.int64) - b.astype(np.int64)"),
    "mean_divides_by_r_minus_1": ("np.divide(acc, np.float32(num_ranks), dtype=np.float32)",
                                  "np.divide(acc, np.float32(max(num_ranks - 1, 1)), dtype=np.float32)"),
    "mean_not_applied": ("        return np.divide(acc, np.float32(num_ranks), dtype=np.float32)",
                         "        return acc"),
    "segments_floor": ("return -(-n // num_ranks)", "return max(n // num_ranks, 1)"),
    "max_is_min": ("out = np.where(a > b, a, b).astype(np.float32)",
                   "out = np.where(a < b, a, b).astype(np.float32)"),
    "i32_max_is_min": ("return np.maximum(a, b)", "return np.minimum(a, b)"),
    "max_nan_ignored": ("bits[np.isnan(a) | np.isnan(b)] = CANONICAL_NAN_BITS", "pass"),
    "max_negative_zero_wins": ("signed_zero = np.where(both_negative, np.float32(-0.0), np.float32(0.0))",
                               "signed_zero = np.where(both_negative, np.float32(0.0), np.float32(-0.0))"),
    "ag_sends_wrong_segment": ("            c = (r - s) % R\n            lo, hi = bounds[c]\n"
                               "            messages.append(((r + 1) % R, c, state[r][lo:hi].copy()))\n"
                               "        for dst, c, received in messages:\n"
                               "            lo, hi = bounds[c]\n            state[dst][lo:hi] = received",
                               "            c = (r - s - 1) % R\n            lo, hi = bounds[c]\n"
                               "            messages.append(((r + 1) % R, c, state[r][lo:hi].copy()))\n"
                               "        for dst, c, received in messages:\n"
                               "            lo, hi = bounds[c]\n            state[dst][lo:hi] = received"),
    "rs_returns_neighbour_shard": ("return [state[r][lo:hi].copy() for r, (lo, hi) in enumerate(bounds)]",
                                   "return [state[(r + 1) % R][lo:hi].copy() for r, (lo, hi) in enumerate(bounds)]"),
    "reduce_reads_root_state": ("result[lo:hi] = state[c][lo:hi]", "result[lo:hi] = state[root][lo:hi]"),
    "all_gather_transposed": ("state[r][lo:hi] = flat[r]", "state[r][lo:hi] = flat[R - 1 - r]"),
    "broadcast_from_rank0": ("src = np.ascontiguousarray(sends[senders[0]])",
                             "src = np.ascontiguousarray(sends[0] if sends[0] is not None else sends[senders[0]]) * 0"),
    "closed_form_starts_at_owner": ("return [(c + k) % num_ranks for k in range(1, num_ranks + 1)]",
                                    "return [(c + k) % num_ranks for k in range(0, num_ranks)]"),
    "closed_form_rank_order": ("return [(c + k) % num_ranks for k in range(1, num_ranks + 1)]",
                               "return list(range(num_ranks))"),
    "closed_form_backwards": ("return [(c + k) % num_ranks for k in range(1, num_ranks + 1)]",
                              "return [(c - k) % num_ranks for k in range(1, num_ranks + 1)]"),
    "at_many_wrong_segment": ("seg = indices // s", "seg = indices // max(s - 1, 1)"),
    "at_wrong_segment": ("c = index // segment_length(n, R)", "c = index // (segment_length(n, R) + 1)"),
    "params_pair_by_position": ("operands = [grads[r][pid] for r in range(R)]",
                                "operands = [list(grads[r].values())[sorted(ids).index(pid)] for r in range(R)]"),
    "params_no_id_check": ("        if set(grads[r]) != ids:\n", "        if False:\n"),
    "params_no_shape_check": ('            raise ParamMismatch("shape", f"parameter {pid}: shape differs between ranks")',
                              "            pass"),
    "params_shape_before_dtype": ("        if any(a.dtype != per_rank[0].dtype for a in per_rank):\n"
                                  '            raise ParamMismatch("dtype"',
                                  "        if any(a.shape != per_rank[0].shape for a in per_rank):\n"
                                  '            raise ParamMismatch("shape"'),
    "params_op_ignored": ("reduced = all_reduce(operands, op)", "reduced = all_reduce(operands, SUM)"),
    "params_rank0_everywhere": ("            out[r][pid] = reduced[r]", "            out[r][pid] = grads[0][pid]"),
    "params_acc_ignored": ("                operands = [accumulate(acc[r][pid], operands[r]) for r in range(R)]",
                           "                pass"),
    "params_acc_from_rank0": ("                operands = [accumulate(acc[r][pid], operands[r]) for r in range(R)]",
                              "                operands = [accumulate(acc[0][pid], operands[r]) for r in range(R)]"),
    "params_acc_partial_accepted": ("            if any(given) and not all(given):", "            if False:"),
    "a2a_transposed": ("out[dst][src * m:(src + 1) * m] = flat[src][dst * m:(dst + 1) * m]",
                       "out[src][dst * m:(dst + 1) * m] = flat[src][dst * m:(dst + 1) * m]"),
    "a2a_wrong_chunk": ("out[dst][src * m:(src + 1) * m] = flat[src][dst * m:(dst + 1) * m]",
                        "out[dst][src * m:(src + 1) * m] = flat[src][src * m:(src + 1) * m]"),
    "a2a_reversed_sources": ("out[dst][src * m:(src + 1) * m] = flat[src][dst * m:(dst + 1) * m]",
                             "out[dst][(R - 1 - src) * m:(R - src) * m] = flat[src][dst * m:(dst + 1) * m]"),
    "gather_list_own_shard": ("return [[np.array(shards[k], copy=True) for k in range(R)] for _ in range(R)]",
                              "return [[np.array(shards[r], copy=True) for k in range(R)] for r in range(R)]"),
    "gather_list_aliases": ("return [[np.array(shards[k], copy=True) for k in range(R)] for _ in range(R)]",
                            "return [[shards[k] for k in range(R)] for _ in range(R)]"),
    "accumulate_averages": ("return combine(_flat(acc), _flat(grad), SUM).reshape(acc.shape)",
                            "return (combine(_flat(acc), _flat(grad), SUM) / np.float32(2)).reshape(acc.shape)"),
    "accumulate_aliases": ("        return grad.copy()", "        return grad"),
    "accumulate_replaces": ("return combine(_flat(acc), _flat(grad), SUM).reshape(acc.shape)",
                            "return grad.copy()"),
    "send_recv_aliases": ("    _check_dtype(x)\n    return x.copy()", "    _check_dtype(x)\n    return x"),
    "reduce_fills_non_roots": ("    out = [None] * R\n    out[root] = result.reshape(shape)",
                               "    out = [result.reshape(shape)] * R"),
    "broadcast_accepts_two_senders": ("    if len(senders) != 1:", "    if len(senders) < 1:"),
    "a2a_accepts_ragged": ('    if n % R:\n        raise OracleError("all_to_all_single input length must be a multiple of R")',
                           "    if False:\n        pass"),
}


def _mutant(name, old, new):
    assert SOURCE.count(old) >= 1, f"mutation {name}: pattern not found in the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SOURCE.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _failing_pins(mod):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_copy_passes():
    mod = types.ModuleType("oracle_copy")
    exec(compile(SOURCE, "<oracle copy>", "exec"), mod.__dict__)
    assert _failing_pins(mod) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    failed = _failing_pins(_mutant(name, old, new))
    assert failed, f"planted mistake {name!r} passed every pin"
