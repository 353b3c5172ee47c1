"""Seeded synthetic workloads for paged-KV decode.

This package only draws random numbers and lays them out; it contains none of
the attention arithmetic. Both the HIP path (through its tests and the bench)
and the CPU oracle read the same arrays from here.
"""

from .configs import (  # noqa: F401
    CONFIG_NAMES,
    BlockTableWorkload,
    GqaWorkload,
    MlaFp8Workload,
    MlaWorkload,
    bf16_bits_from_f32,
    make_block_table,
    make_config,
    make_gqa,
    encode_fp8_rows,
    make_mla,
    make_mla_fp8,
    lognormal_lengths,
)
