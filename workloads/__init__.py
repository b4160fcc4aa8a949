"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This package only draws random inputs and lays them out; it holds none of the
method's arithmetic (no index, score, selection, RoPE or attention code).
"""
from .synth import (CONFIGS, Config, Workload, make_workload, pool_chunks, bf16_bits_to_f32,
                    f32_to_bf16_bits, with_decode_capacity, draw_decode_tokens)

__all__ = ["CONFIGS", "Config", "Workload", "make_workload", "pool_chunks", "bf16_bits_to_f32",
           "f32_to_bf16_bits", "with_decode_capacity", "draw_decode_tokens"]
