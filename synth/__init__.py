"""Seeded synthetic inputs for batched draft verification.

This package is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds none of the verification or estimator arithmetic: it only
draws logits, draft tokens and uniforms, with the shapes and value
distributions of the five workloads described in ``synth.gen``.
"""
from .gen import (  # noqa: F401
    Batch,
    WORKLOADS,
    make_batch,
    workload,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    constant_alpha_rows,
    broadcast_batch,
)
