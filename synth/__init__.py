"""Seeded synthetic THD packs shared by the tests, the smoke check and the bench.

This package only draws inputs: segment lengths and random tensors, rounded once
to the storage dtype. It contains none of the attention method's arithmetic, so
that both the fp64 oracle and the HIP library can consume the very same values.
"""
from .packs import (CONFIGS, CompressorInputs, Layout, Pack, bf16_bits_to_f32, compressor_inputs, f32_to_bf16_bits,
                    make_pack, pack_from_lengths, workload_layout)

__all__ = ["CONFIGS", "CompressorInputs", "Layout", "Pack", "bf16_bits_to_f32", "compressor_inputs",
           "f32_to_bf16_bits", "make_pack", "pack_from_lengths", "workload_layout"]
