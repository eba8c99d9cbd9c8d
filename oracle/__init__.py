"""CPU oracle for the W4A16 linear path.  TEST INFRASTRUCTURE ONLY.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the product library or its binding.
"""
from .w4a16_ref import (  # noqa: F401
    F16, BF16, KOFF_OF_NIBBLE, SLOT_OF_KOFF, SYMMETRIC_ZERO,
    f16_bits_to_f64, bf16_bits_to_f64, act_bits_to_f64,
    f32_to_f16_bits, f32_to_bf16_bits, f32_to_act_bits,
    pack_weights, unpack_weights, pack_zeros, unpack_zeros, slice_of_word, WORDS_PER_RUN,
    word_position, TILE_ROWS,
    dequant_f32, dequant_act, linear_ref, moe_linear_ref,
)
