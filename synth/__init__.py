"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package draws BF16 bit patterns, page tables and sequence lengths. It holds
none of the compression or attention arithmetic.
"""
from .workloads import CONFIGS, Workload, make_workload, f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
