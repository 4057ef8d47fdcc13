"""Seeded synthetic inputs for the paged-decode path.

This package is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It draws random numbers, rounds them to the storage dtypes and lays
out block tables; it holds none of the method's arithmetic (no slab mapping, no
gather, no attention, no quantisation).
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    bits_to_f32,
    device_seed,
    f16_bits_from_f32,
    hadamard_signs,
    kv_bits_for_sequence,
    make_block_table,
    monotone_rows,
    normal_bits,
    normal_device,
    q_bits,
    ranged_bits,
    shuffled_rows,
    workload_lengths,
)
