"""Seeded synthetic THD packs shared by the tests, the smoke check and the bench.

This package only draws inputs: segment lengths and random tensors, rounded once
to the storage dtype. It contains none of the attention method's arithmetic, so
that both the fp64 oracle and the HIP library can consume the very same values.
"""
from .packs import CONFIGS, Pack, make_pack, bf16_bits_to_f32, f32_to_bf16_bits, pack_from_lengths

__all__ = ["CONFIGS", "Pack", "make_pack", "bf16_bits_to_f32", "f32_to_bf16_bits", "pack_from_lengths"]
