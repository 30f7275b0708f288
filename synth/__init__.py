"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This package draws random numbers and stores them in the formats the path
consumes (bf16 bit patterns, fp32, int32).  It holds none of the method's
arithmetic: no quantisation, attention, logits or acceptance.
"""
from .gen import (  # noqa: F401
    TAG, rng, normal_f32, f32_to_bf16_bits, normal_bf16, uniform_f32,
    kept_subset, page_permutation, threads_default,
)
