"""Seeded synthetic inputs for the CSA2 sparse decode path (shared by the HIP path's
tests/bench and by the oracle's tests; holds none of the decode arithmetic)."""
from .generator import (  # noqa: F401
    CONFIGS,
    Workload,
    make_config,
    make_workload,
    make_write_inputs,
    to_paged,
    verify_row_len,
)
