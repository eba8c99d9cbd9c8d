"""Seeded draws of raw W4A16 inputs (no method arithmetic here).

Recipe (one numpy ``default_rng`` stream per case, drawn in this order):
  q     = integers(0, 16, (N, K))            4-bit codes, uniform
  zp    = integers(0, 16, (N, K // group))   asymmetric only, uniform
  s     = |normal(0, 0.02, (N, G))| + 1e-3   float32, then rounded to the act dtype
  bias  = normal(0, 0.1, N)                  only when asked for
  x     = normal(0, 1, (M, K))               float32, then rounded to the act dtype

The rounding of a float32 draw to the activation dtype is the input format's
own conversion (nearest-even): numpy's float16 cast, and torch's bfloat16
cast, whose bit patterns are taken as they come.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

F16 = 0
BF16 = 1


def stream_seed(*parts) -> int:
    """A stable 64-bit seed from any tuple of ints/strings."""
    h = hashlib.sha256(repr(tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little")


def to_act_bits(v: np.ndarray, dtype: int) -> np.ndarray:
    """float32 draws -> activation-dtype bit patterns (uint16)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16)
        return t.numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype}")


@dataclasses.dataclass
class Case:
    M: int
    N: int
    K: int
    group: int
    dtype: int
    q: np.ndarray            # uint8 [N, K], 0..15
    zp: np.ndarray | None    # uint8 [N, G], 0..15, or None (symmetric)
    s_bits: np.ndarray       # uint16 [N, G]
    x_bits: np.ndarray       # uint16 [M, K]
    bias_bits: np.ndarray | None  # uint16 [N] or None

    @property
    def G(self) -> int:
        return self.K // self.group

    @property
    def symmetric(self) -> bool:
        return self.zp is None


def make_case(M: int, N: int, K: int, group: int, dtype: int, symmetric: bool,
              bias: bool, seed, x_seed=None, scale_sigma: float = 0.02,
              scale_floor: float = 1e-3) -> Case:
    """Draw one case.  ``seed`` fixes the weights; ``x_seed`` the activations."""
    if K % group:
        raise ValueError("K must be a multiple of group")
    G = K // group
    rng = np.random.default_rng(stream_seed("w", seed))
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zp = None if symmetric else rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    s = (np.abs(rng.normal(0.0, scale_sigma, size=(N, G))) + scale_floor).astype(np.float32)
    s_bits = to_act_bits(s, dtype)
    bias_bits = None
    if bias:
        bias_bits = to_act_bits(rng.normal(0.0, 0.1, size=N).astype(np.float32), dtype)
    xrng = np.random.default_rng(stream_seed("x", seed if x_seed is None else x_seed, M))
    x_bits = to_act_bits(xrng.normal(0.0, 1.0, size=(M, K)).astype(np.float32), dtype)
    return Case(M, N, K, group, dtype, q, zp, s_bits, x_bits, bias_bits)


def stored_words(seed, first_row: int, rows: int, words_per_row: int) -> np.ndarray:
    """Uniform random uint32 words for rows [first_row, first_row + rows) of a
    packed tensor, drawn in the stored layout itself: uniform words are
    uniform 4-bit codes whatever the nibble order, so a layer too large to
    draw code by code is drawn word by word (one stream per row block)."""
    rng = np.random.default_rng(stream_seed("words", seed, first_row))
    return rng.integers(0, 1 << 32, size=(rows, words_per_row), dtype=np.uint32)
