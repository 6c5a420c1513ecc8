"""CPU oracle for the exact attention forward pass (test infrastructure only).

This package is a plain, slow, float64 statement of what the GPU library
computes.  It is used by the tests, by the smoke check and by the bench's
CPU-baseline leg, and by nothing else: the product path never imports it.
It shares no code with the HIP library; the only thing both sides share is
the seeded input generator in ``workloads``.

Parity pins: every function here is checked against facts fixed by the
pages and by mathematics (closed forms, invariants, brute force, an
independent library routine) in ``tests/test_oracle_pins.py``.
"""
from .exact import (  # noqa: F401
    attention,
    attention_rows,
    attention_bruteforce,
    attention_tiled_online,
    attention_qk,
    attention_backward,
    attention_block_sparse,
    sparse_pair_count,
    pair_count,
    softmax_rows,
    visible_keys,
    unit_flops,
    default_workers,
)
