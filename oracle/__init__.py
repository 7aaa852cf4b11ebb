"""fp64 CPU oracle for paged-KV POD attention.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check and the
benchmark's CPU-baseline leg. The product path (the HIP library and its
Python binding) never imports, links or executes anything in this package.

Functions without an independent pin would be marked "parity unpinned" here;
every function below is pinned by tests/test_oracle.py (closed forms,
invariants, library special cases, hand-worked golden values).
"""
from .attend import (  # noqa: F401
    LN2,
    OracleInputError,
    seq_lens,
    validate_role,
    logical_kv,
    valid_key_mask,
    attend_rows,
    attend_role,
    attend_role_dense,
    merge_states,
    apply_sink,
    e4m3_to_float,
    attend_rows_fp8_scaled,
)
