"""CPU oracle for logical-rank collectives (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does, and this package imports
nothing from it.
"""

from .ring import (  # noqa: F401
    SUM, MEAN, MAX, OPS, CANONICAL_NAN_BITS, OracleError,
    combine, finish, segment_length, segment_bounds, fold_order,
    ring_reduce_scatter_phase, ring_all_gather_phase,
    all_reduce, reduce, broadcast, reduce_scatter, all_gather, all_reduce_many,
    all_reduce_closed_form, all_reduce_at, all_reduce_at_many,
    ParamMismatch, all_reduce_params, accumulate,
    all_gather_list, all_to_all_single, send_recv,
)
