"""Seeded synthetic workloads shared by the tests, the bench and the oracle.

This package only draws inputs (scores, keys, values, sketches, queries) and
rounds them to the storage types; it contains none of the method's
arithmetic, and imports neither the oracle nor the library.
"""

from .gen import (  # noqa: F401
    C5, CONFIGS, bf16_bits, bf16_to_f32, make_decode_workload, make_c5_tau,
    c3_shift_queries, resident_cap,
)
