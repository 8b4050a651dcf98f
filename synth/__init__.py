"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only draws random numbers and shapes them into the workloads the
pages measure (weight matrices and activation matrices of the stated sizes,
distributions and outlier structure). It holds none of the method's arithmetic:
no quantization, no dot products, no rescaling.
"""
from .gen import (  # noqa: F401
    GAMMA, splitmix64, uniform, normal, student_t4, choose_subset,
    bf16_bits, bf16_bits_to_f32, seed_for, Workload, workload, WORKLOADS,
)
