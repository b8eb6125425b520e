"""Seeded synthetic decode workloads shared by the tests, the bench and the smoke check.

This package only draws inputs (bf16 queries, paged bf16 K/V caches, page tables and, for the
hierarchical variant, ground-truth clusters).  It holds none of the method's arithmetic: no
quantisation, no scoring, no softmax, no selection and no attention.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    make_config,
    make_custom,
)
