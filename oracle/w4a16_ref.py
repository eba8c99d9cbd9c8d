"""CPU oracle for the W4A16 linear path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's ``cpu_baseline`` leg
may import this module.  The product path (the HIP library and its Python
binding) never calls it, and this module imports nothing from the product.

What it computes, and where each step comes from (pages by title):

* "[ROCm][Kernel] Add HybridW4A16LinearKernel: Triton prefill + HIP skinny
  decode", description: y = x . dequant(Wq)^T (+bias); 4-bit weights packed
  eight per int32 in an [N, K/8] layout; symmetric ``uint4b8``
  (w = (q - 8) * s) or asymmetric ``uint4`` (w = (q - zp) * s) with per-group
  zero points; group sizes 32, 64 or 128 along K.
* "Upstream sync 67/N: merge 382bbd5144 HybridW4A16LinearKernel (conflict)",
  section "Upstream's Python side is kept -- and it does NOT work here": the
  decode call takes (w_q, x_2d, w_s, cu_count, group_size, w_zp, bias); zero
  points are int32 or uint32 [N/8, groups], eight 4-bit values packed along
  dim 0.
* Word layout (the pages name an "AWQ-style packed shuffle" / "ExLlama
  shuffle" layout [N, K/8] but print no permutation).  Reading used here, in
  two levels:
  - inside a word: the word holding the 8-k slice L of a row stores the
    weight at k = 8*L + KOFF_OF_NIBBLE[t] in the nibble at bit 4*t, with
    KOFF_OF_NIBBLE = (0, 2, 4, 6, 1, 3, 5, 7); equivalently k-offset i lives
    in nibble SLOT_OF_KOFF[i] = (0, 4, 1, 5, 2, 6, 3, 7);
  - across words: each complete run of 16 words (128 k) of a row is a 4x4
    transpose of words -- stored word 4*r + t of the run holds slice 4*t + r
    of the run; a final incomplete run (K not a multiple of 128) keeps its
    slices in order.  ``slice_of_word`` spells the map out;
  - across rows: the rows form tiles of 16 (rows 16*i .. 16*i + 15), and
    every complete tile occupies the 16 * K/8 words starting at word
    16*i * K/8, tile-major: run u of the 16 rows is one block of 256 words
    at offset 256*u, whose word 4*(16*r + j) + e is word 4*r + e of row j's
    run (so the 64 sixteen-byte pieces of a block are ordered (r, j)); the
    incomplete last runs of the 16 rows follow the blocks, row after row.
    A final incomplete tile (N not a multiple of 16) keeps its rows one
    after another, K/8 words each.  ``word_position`` spells the map out.
* Zero-point packing: nibble i (bits 4i..4i+3) of word (r, grp) holds the
  zero point of row 8r + i ("packed 8x uint4 along dim 0").
* Scales: [N, G] row-major in the activation dtype (G = K / group).
* Dequantisation: (q - z) * s is formed exactly in float32 (|q - z| <= 15 has
  4 significant bits, an fp16 scale 11 and a bf16 scale 8, so the product fits
  float32's 24) and rounded once, to nearest-even, to the activation dtype
  only where an activation-dtype weight is asked for (``dequant_act``).
* The product: y = x . W^T + bias accumulated in float64 from the exact
  activation-dtype bits of x, the exact float32 W and the bias bits.

Half-precision values cross this module as raw uint16 bit patterns, because
numpy has no bfloat16 type.

Every function here is pinned by the tests in ``tests/test_oracle_pins.py``
(worked words, round trips, hand-rounded values, exact rational brute force,
closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1

# nibble t of a weight word holds k-offset KOFF_OF_NIBBLE[t] inside its 8-k slice
KOFF_OF_NIBBLE = (0, 2, 4, 6, 1, 3, 5, 7)
# and the inverse: k-offset i is stored in nibble SLOT_OF_KOFF[i]
SLOT_OF_KOFF = (0, 4, 1, 5, 2, 6, 3, 7)

SYMMETRIC_ZERO = 8  # uint4b8: the stored value carries a bias of 8


# --------------------------------------------------------------------------
# half-precision formats (format definitions, no rounding involved)
# --------------------------------------------------------------------------

def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values.

    A bfloat16 is the upper half of a binary32; widening is a 16-bit shift.
    """
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def act_bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F16:
        return f16_bits_to_f64(bits)
    if dtype == BF16:
        return bf16_bits_to_f64(bits)
    raise ValueError(f"unknown activation dtype {dtype}")


def f32_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> binary16, round to nearest, ties to even (numpy's cast)."""
    v = np.asarray(v, dtype=np.float32)
    return v.astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16, round to nearest, ties to even, on the bits.

    Add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.  Only
    finite inputs occur on this path (dequantised weights are bounded by
    15 * max|s|); a NaN or infinity is rejected rather than rounded.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value reached bfloat16 rounding")
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_act_bits(v: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(v)
    if dtype == BF16:
        return f32_to_bf16_bits(v)
    raise ValueError(f"unknown activation dtype {dtype}")


# --------------------------------------------------------------------------
# packing (the layout contract)
# --------------------------------------------------------------------------

WORDS_PER_RUN = 16  # 128 k


def slice_of_word(j: int, words_per_row: int) -> int:
    """Which 8-k slice of its row the stored word j holds.

    Inside a complete run of 16 words the stored order is the 4x4 transpose
    of the slice order (word 4*r + t <-> slice 4*t + r, an involution); an
    incomplete last run is stored in order.
    """
    run, p = divmod(j, WORDS_PER_RUN)
    if (run + 1) * WORDS_PER_RUN <= words_per_row:
        r, t = divmod(p, 4)
        return run * WORDS_PER_RUN + 4 * t + r
    return j


def _word_order(words_per_row: int) -> np.ndarray:
    """order[j] = slice held by stored word j, for one row."""
    return np.array([slice_of_word(j, words_per_row) for j in range(words_per_row)], dtype=np.int64)


TILE_ROWS = 16


def word_position(n: int, j: int, N: int, words_per_row: int) -> int:
    """Flat index, in the packed tensor, of stored word j of row n.

    Rows of a complete 16-row tile are interleaved run by run (block of 256
    words per run, piece order (r, row)); their incomplete runs follow the
    blocks row after row.  Rows of a final incomplete tile are row-major.
    """
    J = words_per_row
    tile, row = divmod(n, TILE_ROWS)
    if (tile + 1) * TILE_ROWS > N:
        return n * J + j
    base = tile * TILE_ROWS * J
    runs = J // WORDS_PER_RUN
    run, p = divmod(j, WORDS_PER_RUN)
    if run < runs:
        r, e = divmod(p, 4)
        return base + 256 * run + 4 * (TILE_ROWS * r + row) + e
    tail = J - runs * WORDS_PER_RUN
    return base + 256 * runs + tail * row + (j - runs * WORDS_PER_RUN)


def _positions(N: int, words_per_row: int) -> np.ndarray:
    """pos[n, j] = word_position(n, j, N, J) for every word, the same cases
    written with whole-array operations."""
    J = words_per_row
    n = np.arange(N, dtype=np.int64)[:, None]
    j = np.arange(J, dtype=np.int64)[None, :]
    tile, row = n // TILE_ROWS, n % TILE_ROWS
    runs = J // WORDS_PER_RUN
    tail = J - runs * WORDS_PER_RUN
    base = tile * TILE_ROWS * J
    run, p = j // WORDS_PER_RUN, j % WORDS_PER_RUN
    in_run = base + 256 * run + 4 * (TILE_ROWS * (p // 4) + row) + p % 4
    in_tail = base + 256 * runs + tail * row + (j - runs * WORDS_PER_RUN)
    tiled = np.where(j < runs * WORDS_PER_RUN, in_run, in_tail)
    complete = (tile + 1) * TILE_ROWS <= N
    return np.where(complete, tiled, n * J + j)


def pack_weights(q: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] with values 0..15 -> int32 [N, K/8] in the word layout."""
    q = np.asarray(q)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("weights must lie in 0..15")
    q8 = q.astype(np.uint32).reshape(N, K // 8, 8)
    by_slice = np.zeros((N, K // 8), dtype=np.uint32)
    for koff in range(8):
        by_slice |= q8[:, :, koff] << np.uint32(4 * SLOT_OF_KOFF[koff])
    # stored word j of a row holds slice order[j]; the word then sits at
    # its position in the row tiles
    stored = by_slice[:, _word_order(K // 8)]
    out = np.empty(N * (K // 8), dtype=np.uint32)
    out[_positions(N, K // 8).ravel()] = stored.ravel()
    return out.reshape(N, K // 8).view(np.int32)


def unpack_weights(wq: np.ndarray) -> np.ndarray:
    """int32 (or uint32) [N, K/8] -> uint8 [N, K]; the bits are unsigned."""
    w = np.asarray(wq).view(np.uint32)
    N, J = w.shape
    stored = w.ravel()[_positions(N, J).ravel()].reshape(N, J)
    by_slice = np.empty_like(stored)
    by_slice[:, _word_order(J)] = stored
    q = np.empty((N, J, 8), dtype=np.uint8)
    for koff in range(8):
        q[:, :, koff] = (by_slice >> np.uint32(4 * SLOT_OF_KOFF[koff])) & np.uint32(0xF)
    return q.reshape(N, J * 8)


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """z uint8 [N, G] with values 0..15 -> int32 [N/8, G], 8 rows per word."""
    z = np.asarray(z)
    N, G = z.shape
    if N % 8:
        raise ValueError("N must be a multiple of 8 to pack zero points")
    if z.size and (z.min() < 0 or z.max() > 15):
        raise ValueError("zero points must lie in 0..15")
    z8 = z.astype(np.uint32).reshape(N // 8, 8, G)
    word = np.zeros((N // 8, G), dtype=np.uint32)
    for i in range(8):
        word |= z8[:, i, :] << np.uint32(4 * i)
    return word.view(np.int32)


def unpack_zeros(zpk: np.ndarray) -> np.ndarray:
    """int32 (or uint32) [N/8, G] -> uint8 [N, G]."""
    w = np.asarray(zpk).view(np.uint32)
    R, G = w.shape
    z = np.empty((R, 8, G), dtype=np.uint8)
    for i in range(8):
        z[:, i, :] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return z.reshape(R * 8, G)


# --------------------------------------------------------------------------
# dequantisation and the product
# --------------------------------------------------------------------------

def _zero_points(zpk, N: int, G: int) -> np.ndarray:
    if zpk is None:
        return np.full((N, G), SYMMETRIC_ZERO, dtype=np.uint8)
    z = unpack_zeros(zpk)
    if z.shape != (N, G):
        raise ValueError(f"zero points unpack to {z.shape}, expected {(N, G)}")
    return z


def dequant_f32(wq, scale_bits, zpk, N: int, K: int, group: int, dtype: int) -> np.ndarray:
    """Exact dequantised weights W[n, k] = (q - z[n, k//g]) * s[n, k//g], float32."""
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    q = unpack_weights(wq)
    if q.shape != (N, K):
        raise ValueError(f"weights unpack to {q.shape}, expected {(N, K)}")
    z = _zero_points(zpk, N, G)
    s = act_bits_to_f64(np.asarray(scale_bits).reshape(N, G), dtype)
    # group index of every k, spelled out
    grp = np.arange(K) // group
    diff = q.astype(np.int32) - z[:, grp].astype(np.int32)
    w64 = diff.astype(np.float64) * s[:, grp]
    w32 = w64.astype(np.float32)
    # the product is exact in float32; check that the narrowing lost nothing
    if not np.array_equal(w32.astype(np.float64), w64):
        raise AssertionError("dequantised product is not exact in float32")
    return w32


def dequant_act(wq, scale_bits, zpk, N: int, K: int, group: int, dtype: int) -> np.ndarray:
    """Dequantised weights rounded once (nearest-even) to the activation dtype, as bits."""
    return f32_to_act_bits(dequant_f32(wq, scale_bits, zpk, N, K, group, dtype), dtype)


def linear_ref(x_bits, wq, scale_bits, zpk, bias_bits, M: int, N: int, K: int,
               group: int, dtype: int) -> np.ndarray:
    """y[M, N] = x . W^T (+ bias), accumulated in float64 from the exact inputs."""
    x = act_bits_to_f64(np.asarray(x_bits).reshape(M, K), dtype)
    w = dequant_f32(wq, scale_bits, zpk, N, K, group, dtype).astype(np.float64)
    y = x @ w.T
    if bias_bits is not None:
        y = y + act_bits_to_f64(np.asarray(bias_bits).reshape(N), dtype)[None, :]
    return y



# --------------------------------------------------------------------------
# expert-indexed product (fused MoE skinny GEMM)
# --------------------------------------------------------------------------

def moe_linear_ref(x_bits, wq, scale_bits, zpk, bias_bits, topk_ids, topk_weights,
                   M: int, topk: int, E: int, N: int, K: int, group: int, dtype: int,
                   x_per_slot: bool = False) -> np.ndarray:
    """Expert-indexed product, one output row per (token, slot), float64.

    The pages name a fused-MoE variant of the skinny kernel (an expert-indexed
    W4A16 GEMM; "Upstream sync 67/N: merge 382bbd5144 HybridW4A16LinearKernel
    (conflict)", conflict table) without printing its contract.  Reading used:
    slot s = m * topk + j of token m uses expert e = topk_ids[m, j], whose
    weights, scales, zero points and bias are slice e of stacks [E, ...] in the
    linear layer's layouts, and
        y[s] = topk_weights[m, j] * (x_row . W_e^T + b_e)
    with x_row = x[m] (x of shape [M, K]) or x[s] (x of shape [M*topk, K]);
    no weights means 1.  An id outside [0, E) gives a zero row.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(M, topk)
    x = np.asarray(x_bits).reshape(M * topk if x_per_slot else M, K)
    wq = np.asarray(wq).reshape(E, N, K // 8)
    s = np.asarray(scale_bits).reshape(E, N, K // group)
    z = None if zpk is None else np.asarray(zpk).reshape(E, N // 8, K // group)
    b = None if bias_bits is None else np.asarray(bias_bits).reshape(E, N)
    y = np.zeros((M * topk, N), dtype=np.float64)
    for m in range(M):
        for j in range(topk):
            slot = m * topk + j
            e = int(ids[m, j])
            if not 0 <= e < E:
                continue
            row = x[slot if x_per_slot else m][None, :]
            y[slot] = linear_ref(row, wq[e], s[e], None if z is None else z[e],
                                 None if b is None else b[e], 1, N, K, group, dtype)[0]
            if topk_weights is not None:
                y[slot] *= float(np.asarray(topk_weights, dtype=np.float32).reshape(M, topk)[m, j])
    return y
