"""Seeded synthetic decode workloads shared by the tests, the benchmark and smoke().

This package only draws inputs (random values, context lengths, block tables,
slot mappings).  It holds none of the attention arithmetic: neither the GPU
path nor the CPU oracle is imported here, and both consume what it returns.
"""
from .prefill import (PrefillBatch, llama7b_prefill_chunks, llama7b_prefill_long,  # noqa: F401
                      poison_prefill, prefill_batch)
from .synth import (  # noqa: F401
    Workload,
    CONFIGS,
    make,
    worked_example,
    llama7b_mha,
    gqa,
    long_context,
    fp8_shared_prefix,
    poison_unused_slots,
    to_numpy_bits,
)
