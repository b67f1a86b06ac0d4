"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package draws random numbers and shapes them into the workloads the
recurrence is run on. It performs none of the recurrence's arithmetic, so both
the HIP path and the CPU oracle can consume its output without sharing code.
"""
from .workloads import (  # noqa: F401
    Workload,
    bf16_round,
    draw_varlen_lengths,
    make_prefill,
    make_decode,
    make_product,
    make_product_decode,
    preset,
    PRESETS,
)
