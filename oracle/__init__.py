"""fp64 CPU oracle for AKV drop / repos / splice / compaction / segment-batch
attention.

TEST INFRASTRUCTURE ONLY: imported by `tests/`, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py`, never by the product package
`kv_cache_drop_amd`.  It shares no code with the HIP path.
"""
from .akv_oracle import (  # noqa: F401
    DEFAULT_COMPACT_THRESHOLD, EInval, ENoMem, ERange, EState, OracleError, Pool,
    dense_masked_attention, page_mass, rope_inv_freq, rotate, segment_attention,
)
from .script import OracleRun, apply_op, run_workload, segment_lists  # noqa: F401
