"""Seeded synthetic inputs for the sparse FP8 MLA decode path.

This package only draws random inputs and lays their bytes out in the
``fp8_ds_mla`` page format.  It holds none of the decode arithmetic (no
dequantisation, no attention, no index resolution), so both the CPU oracle
and the HIP path can consume what it produces without sharing any code.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    D_QK,
    D_NOPE,
    D_ROPE,
    ROW_DATA_BYTES,
    ROW_SCALE_BYTES,
    ROW_BYTES,
    Workload,
    make_workload,
    make_code_sweep,
    make_custom,
    make_writer_rows,
    poison_rows,
    split_swa_pool,
    workload_digest,
)
