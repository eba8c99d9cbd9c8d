"""Seeded synthetic inputs for the W4A16 linear path.

This package draws raw inputs only: 4-bit codes, zero points, scales,
activations and biases, with the value distributions of the workloads the
W4A16 pages tune on (Qwen3-4B and Llama-3.1-8B layer shapes).  It holds none
of the method's arithmetic: no packing, no dequantisation, no product.  Both
the CPU oracle side and the GPU side of every test take their inputs from
here; half-precision values are handed over as raw uint16 bit patterns.
"""
from .gen import Case, make_case, to_act_bits, stream_seed, stored_words  # noqa: F401
from .configs import CONFIGS, Layer, config_cases  # noqa: F401
