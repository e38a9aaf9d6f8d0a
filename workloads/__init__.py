"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package draws random numbers and lays them out in the shapes the attention
path consumes.  It contains none of the method's arithmetic (no normalisation,
rotation, softmax or matrix products), so both the HIP path and the CPU oracle
can be fed from it without sharing any computation.
"""

from .synth import (  # noqa: F401
    HeadConfig,
    PrefillInputs,
    DecodeInputs,
    AppendInputs,
    NormInputs,
    NextTokenInputs,
    WorkloadInputs,
    WORKLOADS,
    build_workload,
    make_prefill_inputs,
    prefill_inputs_from_rows,
    make_decode_inputs,
    make_append_inputs,
    make_norm_inputs,
    make_next_token_inputs,
    PagedCache,
    make_block_table,
    paged_from_contiguous,
    qkv_width,
)
