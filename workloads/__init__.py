"""Seeded synthetic inputs for the CSA/HCA compressed-KV attention step.

This package holds the workload shapes and the seeded random generators that
both the CPU oracle's tests and the GPU path's tests/bench draw from.  It holds
none of the method's arithmetic: it only draws numbers and rounds the draws to
the storage types (bf16 bit patterns, int8, packed FP4 codes, FP8 E4M3 codes).
"""
from .configs import WORKLOADS, Workload, get
from .gen import (
    seed_of,
    rng,
    bf16_normal,
    int8_uniform,
    ragged_lengths,
    bf16_bits_from_f32,
    device_bf16_normal,
    device_int8_uniform,
    fp4_uniform,
    device_fp4_uniform,
    fp8_e4m3_bits,
    kv8_rows,
    kv8_normal,
    device_kv8_normal,
)

__all__ = [
    "WORKLOADS", "Workload", "get", "seed_of", "rng", "bf16_normal", "int8_uniform",
    "ragged_lengths", "bf16_bits_from_f32", "device_bf16_normal", "device_int8_uniform",
    "fp4_uniform", "device_fp4_uniform",
    "fp8_e4m3_bits", "kv8_rows", "kv8_normal", "device_kv8_normal",
]
