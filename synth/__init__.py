"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package draws random numbers and shapes them (row normalisation,
rounding to bf16); it holds none of the decode arithmetic. The oracle and the
HIP library both receive what it produces and neither imports the other.
"""

from .inputs import (  # noqa: F401
    Workload,
    WORKLOADS,
    make_inputs,
    make_cache_device,
    round_bf16,
    bf16_bits,
    ragged_lens,
    fp8_codes,
    fp8_scale,
    fp8_inputs,
    fp8_device,
)
