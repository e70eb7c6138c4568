"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py.

This package only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no hashing, merging, pruning or
attention), so both the oracle and the HIP path can take their inputs from it
without sharing any computation.
"""

from .workloads import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    make_workload,
    round_to_dtype,
    bf16_bits,
    gaussian,
)
