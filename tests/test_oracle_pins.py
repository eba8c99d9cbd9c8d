"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle function to something fixed independently of it:
hand-packed words (worked from the layout stated in the oracle's header),
hand-rounded values, exact rational arithmetic, closed forms, invariants, or
an independent library conversion.  They are chosen so that a plausible slip
(a swapped nibble order, a wrong group index, a dropped bias, a sign error, a
transposed operand, truncation instead of nearest-even) fails at least one.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from synth import make_case

# --------------------------------------------------------------------------
# independent decoders of the half formats (by hand, from the bit fields)
# --------------------------------------------------------------------------


def _frac_from_fields(bits: int, ebits: int, mbits: int) -> Fraction:
    sign = -1 if (bits >> (ebits + mbits)) & 1 else 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    bias = (1 << (ebits - 1)) - 1
    assert e != (1 << ebits) - 1, "inf/nan not expected"
    if e == 0:
        return sign * Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    return sign * (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)


def frac_f16(bits: int) -> Fraction:
    return _frac_from_fields(int(bits), 5, 10)


def frac_bf16(bits: int) -> Fraction:
    return _frac_from_fields(int(bits), 8, 7)


def frac_act(bits, dtype):
    return frac_f16(bits) if dtype == O.F16 else frac_bf16(bits)


def test_half_decoders_exhaustive():
    # every finite bit pattern of both formats decodes to the value its bit
    # fields define (sign, biased exponent, hidden bit, subnormals)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dec, frac, ebits, mbits in ((O.f16_bits_to_f64, frac_f16, 5, 10),
                                    (O.bf16_bits_to_f64, frac_bf16, 8, 7)):
        e = (allbits.astype(np.uint32) >> mbits) & ((1 << ebits) - 1)
        finite = allbits[e != (1 << ebits) - 1]
        vals = dec(finite)
        for b, v in zip(finite[::3], vals[::3]):
            assert Fraction(float(v)) == frac(int(b))


# --------------------------------------------------------------------------
# packing: worked words
# --------------------------------------------------------------------------
# Layout (oracle header): nibble t of a word holds k-offset (0,2,4,6,1,3,5,7)[t].
# So for q = [q0..q7] the word, written as nibbles 7..0 (most significant
# first), reads  q7 q5 q3 q1 q6 q4 q2 q0.


def _word(q8):
    return int(O.pack_weights(np.array([q8], dtype=np.uint8))[0, 0]) & 0xFFFFFFFF


def test_worked_words_weights():
    # q = 0..7: nibbles (msb..lsb) 7 5 3 1 6 4 2 0
    assert _word(list(range(8))) == 0x75316420
    # q = 8..15: nibbles F D B 9 E C A 8; as int32 this is negative
    assert _word(list(range(8, 16))) == 0xFDB9ECA8
    assert int(O.pack_weights(np.array([list(range(8, 16))], dtype=np.uint8))[0, 0]) == -38146904
    assert _word([8] * 8) == 0x88888888
    assert _word([1, 0, 0, 0, 0, 0, 0, 0]) == 0x00000001
    assert _word([0, 1, 0, 0, 0, 0, 0, 0]) == 0x00010000
    assert _word([0, 0, 1, 0, 0, 0, 0, 0]) == 0x00000010
    assert _word([0, 0, 0, 0, 0, 0, 0, 1]) == 0x10000000


def test_worked_words_pairs_fall_in_16bit_halves():
    # the point of this order: shifting a word right by 4*i and masking with
    # 0x000F000F leaves the consecutive pair (k=2i, k=2i+1) in the low and high
    # 16-bit halves.  Checked on the packed word of q = 0..7.
    w = _word(list(range(8)))
    for i in range(4):
        pair = (w >> (4 * i)) & 0x000F000F
        assert pair & 0xF == 2 * i
        assert pair >> 16 == 2 * i + 1


def test_worked_words_two_words_and_rows():
    q = np.zeros((2, 16), dtype=np.uint8)
    q[0, 8] = 3           # row 0, word 1, k-offset 0 -> nibble 0
    q[1, 15] = 5          # row 1, word 1, k-offset 7 -> nibble 7
    w = O.pack_weights(q).view(np.uint32)
    assert w.tolist() == [[0, 0x3], [0, 0x50000000]]


def test_worked_words_runs_of_128_k():
    # a row of K = 128 is one complete run of 16 words, stored as the 4x4
    # transpose of its slices: stored word 4*r + t holds slice 4*t + r.
    def stored_words(k_hot, K=128, val=1):
        q = np.zeros((1, K), dtype=np.uint8)
        q[0, k_hot] = val
        return O.pack_weights(q).view(np.uint32)[0].tolist()
    w = stored_words(8)          # slice 1 = 4*0 + 1 -> t=0, r=1 -> word 4
    assert [j for j, v in enumerate(w) if v] == [4] and w[4] == 0x1
    w = stored_words(32)         # slice 4 = 4*1 + 0 -> t=1, r=0 -> word 1
    assert [j for j, v in enumerate(w) if v] == [1] and w[1] == 0x1
    w = stored_words(127, val=7)  # slice 15 stays at word 15; k-offset 7 -> nibble 7
    assert [j for j, v in enumerate(w) if v] == [15] and w[15] == 0x70000000
    w = stored_words(8 * 6 + 1, val=3)  # slice 6 = 4*1 + 2 -> word 4*2 + 1 = 9; k-offset 1 -> nibble 4
    assert [j for j, v in enumerate(w) if v] == [9] and w[9] == 0x30000
    # K = 160: one complete run and an incomplete one (4 words, stored in order)
    w = stored_words(128 + 8 * 3 + 2, K=160, val=5)   # slice 19 -> word 19; k-offset 2 -> nibble 1
    assert [j for j, v in enumerate(w) if v] == [19] and w[19] == 0x50
    # the map itself: an involution on complete runs, the identity on the rest
    for J in (16, 20, 48):
        order = [O.slice_of_word(j, J) for j in range(J)]
        assert sorted(order) == list(range(J))
        assert all(O.slice_of_word(order[j], J) == j for j in range(J))
    assert [O.slice_of_word(j, 20) for j in range(16, 20)] == [16, 17, 18, 19]


def test_worked_words_row_tiles():
    # rows form tiles of 16; a complete tile stores run u of its rows as one
    # 256-word block, word 4*(16*r + j) + e = word 4*r + e of row j's run;
    # incomplete runs follow row after row; a final incomplete tile is
    # row-major.  Each case: one nonzero code, its flat word index and value.
    def hot(N, K, n, k, val=1):
        q = np.zeros((N, K), dtype=np.uint8)
        q[n, k] = val
        w = O.pack_weights(q).view(np.uint32).ravel()
        nz = [i for i, v in enumerate(w) if v]
        assert len(nz) == 1
        return nz[0], int(w[nz[0]])
    # N=16, K=128: one tile, one run
    assert hot(16, 128, 3, 8) == (76, 0x1)          # slice 1 -> run word 4 (r=1, e=0) -> 4*(16+3)
    assert hot(16, 128, 0, 32) == (1, 0x1)          # slice 4 -> run word 1 (r=0, e=1)
    assert hot(16, 128, 15, 127, 7) == (255, 0x70000000)  # slice 15 -> run word 15 -> 4*(48+15)+3
    assert hot(16, 128, 8, 49, 3) == (161, 0x30000)  # slice 6 -> run word 9 (r=2, e=1) -> 4*(32+8)+1
    # N=16, K=160: the incomplete run (4 words a row) after the block
    assert hot(16, 160, 5, 128 + 8 * 3 + 2, 5) == (279, 0x50)  # 256 + 4*5 + 3
    # N=16, K=256: second run's block
    assert hot(16, 256, 2, 128 + 8) == (328, 0x1)    # 256 + 4*(16*1 + 2)
    # N=32, K=128: second tile starts at word 16*16
    assert hot(32, 128, 16, 0) == (256, 0x1)
    assert hot(32, 128, 17, 32) == (261, 0x1)       # 256 + 4*(0 + 1) + 1
    # N=24, K=128: rows 16..23 are an incomplete tile, row-major
    assert hot(24, 128, 17, 8) == (17 * 16 + 4, 0x1)
    assert hot(24, 128, 0, 0) == (0, 0x1)
    # a 16-byte piece of a block holds one row's slices r, 4+r, 8+r, 12+r
    q = np.zeros((16, 128), dtype=np.uint8)
    for sl in (2, 6, 10, 14):
        q[7, 8 * sl] = 1 + sl // 4
    w = O.pack_weights(q).view(np.uint32).ravel()
    piece = 16 * 2 + 7
    assert w[4 * piece:4 * piece + 4].tolist() == [1, 2, 3, 4]
    assert int(np.count_nonzero(w)) == 4
    # word_position is a bijection onto the tensor for ragged shapes too, and
    # the whole-array map the packer uses agrees with it word for word
    from oracle.w4a16_ref import _positions
    for N, J in ((16, 16), (16, 20), (32, 44), (40, 28), (7, 20), (48, 4), (33, 64)):
        pos = [O.word_position(n, j, N, J) for n in range(N) for j in range(J)]
        assert sorted(pos) == list(range(N * J))
        assert _positions(N, J).ravel().tolist() == pos


def test_worked_words_zeros():
    z = np.arange(8, dtype=np.uint8).reshape(8, 1)
    assert int(O.pack_zeros(z).view(np.uint32)[0, 0]) == 0x76543210
    z = np.zeros((16, 2), dtype=np.uint8)
    z[9, 1] = 0xF        # word row 1, group 1, nibble 1
    w = O.pack_zeros(z).view(np.uint32)
    assert w.tolist() == [[0, 0], [0, 0xF0]]


def test_unpack_of_signed_words_is_logical():
    # int32 -38146904 is the word 0xFDB9ECA8; unpacking must not sign-extend
    w = np.array([[-38146904]], dtype=np.int32)
    assert O.unpack_weights(w).tolist() == [list(range(8, 16))]
    z = np.array([[np.int32(-1)]], dtype=np.int32)
    assert O.unpack_zeros(z).ravel().tolist() == [15] * 8


def test_round_trips():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, (24, 96), dtype=np.uint8)
    assert np.array_equal(O.unpack_weights(O.pack_weights(q)), q)
    words = rng.integers(0, 2**32, (5, 7), dtype=np.uint64).astype(np.uint32).view(np.int32)
    assert np.array_equal(O.pack_weights(O.unpack_weights(words)), words)
    z = rng.integers(0, 16, (32, 5), dtype=np.uint8)
    assert np.array_equal(O.unpack_zeros(O.pack_zeros(z)), z)
    zw = rng.integers(0, 2**32, (4, 3), dtype=np.uint64).astype(np.uint32).view(np.int32)
    assert np.array_equal(O.pack_zeros(O.unpack_zeros(zw)), zw)


def test_pack_rejects_bad_shapes_and_values():
    with pytest.raises(ValueError):
        O.pack_weights(np.zeros((2, 12), dtype=np.uint8))
    with pytest.raises(ValueError):
        O.pack_weights(np.full((1, 8), 16, dtype=np.uint8))
    with pytest.raises(ValueError):
        O.pack_zeros(np.zeros((12, 2), dtype=np.uint8))


# --------------------------------------------------------------------------
# rounding and dequantisation: hand-rounded values
# --------------------------------------------------------------------------


def _dq_one(qv, zv, s_bits, dtype):
    """Dequantise a single weight through the oracle (one 8-weight word, g=8 is
    not allowed by the library but the oracle's arithmetic does not care)."""
    q = np.full((8, 8), zv, dtype=np.uint8)
    q[0, 0] = qv
    wq = O.pack_weights(q)
    z = np.full((8, 1), zv, dtype=np.uint8)
    s = np.full((8, 1), s_bits, dtype=np.uint16)
    out = O.dequant_act(wq, s, O.pack_zeros(z), 8, 8, 8, dtype)
    return int(out[0, 0]), int(out[0, 1])


def test_worked_dequant_fp16():
    # s = fp16 0x251F = 0.0200042724609375; 7 * s = 0.1400299072265625 exactly,
    # the nearest fp16 values are 0x307B = 0.1400146484375 and 0x307C = 0.14013671875;
    # the first is nearer.
    assert frac_f16(0x251F) * 7 == Fraction(1400299072265625, 10**16)
    assert _dq_one(15, 8, 0x251F, O.F16)[0] == 0x307B
    # tie: s = 0x3C03 (1 + 3/1024), 3 * s = 3.0087890625 lies halfway between
    # 0x4204 (3.0078125, even) and 0x4205 (3.009765625): nearest-even picks 0x4204
    assert frac_f16(0x3C03) * 3 == (frac_f16(0x4204) + frac_f16(0x4205)) / 2
    assert _dq_one(11, 8, 0x3C03, O.F16)[0] == 0x4204
    # q = z gives +0 (and so does every other weight of the row here)
    assert _dq_one(5, 5, 0x3C03, O.F16) == (0x0000, 0x0000)


def test_worked_dequant_bf16():
    # s = bf16 0x3CA4 = 0.02001953125; 7 * s = 0.14013671875 exactly; bf16
    # neighbours 0x3E0F = 0.139648.. and 0x3E10 = 0.140625: the second is nearer
    assert frac_bf16(0x3CA4) * 7 == Fraction(14013671875, 10**11)
    assert _dq_one(15, 8, 0x3CA4, O.BF16)[0] == 0x3E10
    # tie: s = 0x3F83 (1 + 3/128), 3 * s = 3.0703125, halfway between 0x4044
    # (3.0625, even mantissa) and 0x4045 (3.078125)
    assert frac_bf16(0x3F83) * 3 == (frac_bf16(0x4044) + frac_bf16(0x4045)) / 2
    assert _dq_one(3, 0, 0x3F83, O.BF16)[0] == 0x4044
    # negative: (0 - 15) * s rounds symmetrically
    neg = _dq_one(0, 15, 0x3CA4, O.BF16)[0]
    assert frac_bf16(neg) == -frac_bf16(_dq_one(15, 0, 0x3CA4, O.BF16)[0])


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.normal(0, 1, 20000).astype(np.float32),
        rng.normal(0, 1e-30, 1000).astype(np.float32),      # bf16 subnormal range
        # exact ties: low 16 bits 0x8000, both parities of the kept lsb
        (np.arange(2000, dtype=np.uint32) * 0x10000 + 0x3F800000 + 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.0703125, 65504.0], dtype=np.float32),
    ])
    mine = O.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_fp16_rounding_matches_exact_nearest_even():
    # brute force on a grid that includes ties: every value k/2048 in [2, 4)
    # sits on the fp16 grid (ulp 1/512) or on a quarter/half point of it
    vals = np.arange(2 * 2048, 4 * 2048, dtype=np.float64) / 2048.0
    bits = O.f32_to_f16_bits(vals.astype(np.float32))
    for v, b in zip(vals[::7], bits[::7]):
        fv = Fraction(v)
        lo = (fv * 512).__floor__()
        cand = [Fraction(lo, 512), Fraction(lo + 1, 512)]
        d = [abs(c - fv) for c in cand]
        if d[0] < d[1] or (d[0] == d[1] and lo % 2 == 0):
            want = cand[0]
        else:
            want = cand[1]
        assert frac_f16(b) == want


def test_dequant_exhaustive_small_codes_against_fractions():
    # every (q, z) pair, a spread of scales, both dtypes: the oracle's float32
    # product equals the exact rational product, and its rounding is the
    # nearest-even neighbour of that rational
    rng = np.random.default_rng(3)
    for dtype in (O.F16, O.BF16):
        for s_f in rng.uniform(1e-3, 0.08, 6).astype(np.float32):
            s_bits = int((O.f32_to_f16_bits if dtype == O.F16 else O.f32_to_bf16_bits)(np.array([s_f]))[0])
            sv = frac_act(s_bits, dtype)
            q = np.tile(np.arange(16, dtype=np.uint8), (16, 1))       # [z, q] grid on rows
            z = np.arange(16, dtype=np.uint8).reshape(16, 1)
            wq = O.pack_weights(q)
            s = np.full((16, 1), s_bits, dtype=np.uint16)
            w32 = O.dequant_f32(wq, s, O.pack_zeros(z), 16, 16, 16, dtype)
            wact = O.dequant_act(wq, s, O.pack_zeros(z), 16, 16, 16, dtype)
            for zi in range(16):
                for qi in range(16):
                    exact = (qi - zi) * sv
                    assert Fraction(float(w32[zi, qi])) == exact
                    got = frac_act(int(wact[zi, qi]), dtype)
                    # nearest: no representable value strictly closer.  Check
                    # against the two neighbours of `got` in the format.
                    b = int(wact[zi, qi])
                    if got == 0:
                        assert exact == 0
                        continue
                    up = frac_act(b + 1, dtype)
                    dn = frac_act(b - 1, dtype) if (b & 0x7FFF) else -up
                    assert abs(got - exact) <= abs(up - exact)
                    assert abs(got - exact) <= abs(dn - exact)


# --------------------------------------------------------------------------
# the product: exact rational brute force on tiny shapes
# --------------------------------------------------------------------------


def _brute_force(case):
    """y from the RAW draws (q, z, s, x, bias), never from packed words.

    Returns the exact rational y and the exact sum of |x * w| per output,
    which bounds the float64 round-off of any summation order.
    """
    G = case.G
    s = [[frac_act(case.s_bits[n, j], case.dtype) for j in range(G)] for n in range(case.N)]
    x = [[frac_act(case.x_bits[m, k], case.dtype) for k in range(case.K)] for m in range(case.M)]
    out, mags = [], []
    for m in range(case.M):
        row, mrow = [], []
        for n in range(case.N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(case.K):
                j = k // case.group
                z = 8 if case.zp is None else int(case.zp[n, j])
                t = x[m][k] * (int(case.q[n, k]) - z) * s[n][j]
                acc += t
                mag += abs(t)
            if case.bias_bits is not None:
                b = frac_act(case.bias_bits[n], case.dtype)
                acc += b
                mag += abs(b)
            row.append(acc)
            mrow.append(mag)
        out.append(row)
        mags.append(mrow)
    return out, mags


def _oracle_y(case):
    zpk = None if case.zp is None else O.pack_zeros(case.zp)
    return O.linear_ref(case.x_bits, O.pack_weights(case.q), case.s_bits, zpk, case.bias_bits,
                        case.M, case.N, case.K, case.group, case.dtype)


@pytest.mark.parametrize("dtype", [O.F16, O.BF16])
@pytest.mark.parametrize("sym,bias", [(True, False), (False, True), (False, False), (True, True)])
@pytest.mark.parametrize("shape", [(1, 8, 64, 32), (3, 16, 64, 32), (2, 8, 96, 32)])
def test_linear_ref_brute_force(dtype, sym, bias, shape):
    M, N, K, g = shape
    case = make_case(M, N, K, g, dtype, sym, bias, seed=("bf", M, N, K, g, dtype, sym, bias))
    exact, mags = _brute_force(case)
    y = _oracle_y(case)
    eps = Fraction(1, 2**53)
    for m in range(M):
        for n in range(N):
            # a float64 sum of K+1 terms is off by at most (K+1) * eps * sum|terms|
            assert abs(Fraction(float(y[m, n])) - exact[m][n]) <= (K + 1) * eps * mags[m][n]


def test_linear_ref_group_boundaries_matter():
    # a case where a wrong group index (k % G instead of k // g) changes y:
    # two groups with very different scales
    case = make_case(1, 8, 64, 32, O.F16, False, False, seed="groups")
    case.s_bits[:, 0] = 0x3C00   # 1.0
    case.s_bits[:, 1] = 0x4000   # 2.0
    exact, _ = _brute_force(case)
    y = _oracle_y(case)
    for n in range(8):
        assert abs(Fraction(float(y[0, n])) - exact[0][n]) < Fraction(1, 10**9)


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------


def test_all_eights_symmetric_is_exactly_zero_or_bias():
    case = make_case(3, 16, 128, 32, O.BF16, True, True, seed="z8")
    case.q[:] = 8
    y = _oracle_y(case)
    b = O.bf16_bits_to_f64(case.bias_bits)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))
    case.bias_bits = None
    y = _oracle_y(case)
    assert np.all(y == 0) and not np.any(np.signbit(y))


def test_asymmetric_q_equal_z_is_zero():
    case = make_case(2, 16, 64, 32, O.F16, False, False, seed="qz")
    case.q[:] = np.repeat(case.zp, 32, axis=1)
    assert np.all(_oracle_y(case) == 0)


def test_closed_form_ones_times_nine():
    # x = 1, symmetric, q = 9: every weight is s, so y[n] = g * sum_j s[n, j] + bias
    case = make_case(1, 16, 256, 64, O.F16, True, True, seed="cf")
    case.q[:] = 9
    case.x_bits[:] = 0x3C00
    y = _oracle_y(case)
    s = O.f16_bits_to_f64(case.s_bits)
    want = 64 * s.sum(axis=1) + O.f16_bits_to_f64(case.bias_bits)
    assert np.allclose(y[0], want, rtol=0, atol=1e-12)


def test_one_hot_x_picks_a_dequantised_weight():
    case = make_case(1, 16, 128, 32, O.BF16, False, False, seed="oh")
    W = O.dequant_f32(O.pack_weights(case.q), case.s_bits, O.pack_zeros(case.zp),
                      16, 128, 32, O.BF16)
    for k in (0, 1, 7, 8, 31, 32, 77, 127):
        case.x_bits[:] = 0
        case.x_bits[0, k] = 0x3F80   # bf16 1.0
        y = _oracle_y(case)
        assert np.array_equal(y[0], W[:, k].astype(np.float64))
        # and this is the weight brute force gives
        z = case.zp[:, k // 32].astype(np.int64)
        sv = O.bf16_bits_to_f64(case.s_bits[:, k // 32])
        assert np.array_equal(y[0], (case.q[:, k].astype(np.int64) - z) * sv)


def test_symmetric_equals_asymmetric_with_zero_eight():
    case = make_case(2, 16, 128, 32, O.F16, True, True, seed="se")
    y_sym = _oracle_y(case)
    case.zp = np.full((16, 4), 8, dtype=np.uint8)
    y_asym = _oracle_y(case)
    assert np.array_equal(y_sym, y_asym)


def test_power_of_two_scale_linearity():
    case = make_case(2, 16, 128, 64, O.BF16, False, False, seed="lin")
    y = _oracle_y(case)
    s = O.bf16_bits_to_f64(case.s_bits).astype(np.float32) * np.float32(4.0)
    case.s_bits = O.f32_to_bf16_bits(s)
    assert np.array_equal(_oracle_y(case), 4.0 * y)


def test_additivity_over_k_halves():
    # y over the whole K equals the sum of y over the two group-aligned halves
    # (a dropped term, or a group index that does not follow k, breaks this)
    case = make_case(2, 16, 256, 64, O.BF16, False, False, seed="kadd")
    y = _oracle_y(case)
    halves = []
    for lo, hi in ((0, 128), (128, 256)):
        q = case.q[:, lo:hi]
        zp = case.zp[:, lo // 64:hi // 64]
        s = case.s_bits[:, lo // 64:hi // 64]
        x = case.x_bits[:, lo:hi]
        halves.append(O.linear_ref(x, O.pack_weights(q), s, O.pack_zeros(zp), None,
                                   2, 16, 128, 64, O.BF16))
    assert np.allclose(y, halves[0] + halves[1], rtol=1e-13, atol=1e-13)


def test_row_permutation_equivariance():
    case = make_case(2, 16, 64, 32, O.F16, False, True, seed="perm")
    y = _oracle_y(case)
    p = np.random.default_rng(5).permutation(16)
    case.q = case.q[p]
    case.zp = case.zp[p]
    case.s_bits = case.s_bits[p]
    case.bias_bits = case.bias_bits[p]
    assert np.array_equal(_oracle_y(case), y[:, p])


def test_per_channel_equals_groups_with_one_scale_per_row():
    # group = K (one scale and zero point per row) is the same layer as any
    # smaller group whose scales and zero points repeat along the row
    for dt, sym in ((O.BF16, False), (O.F16, True)):
        c = make_case(3, 16, 384, 384, dt, sym, True, seed=("perchan", dt, sym))
        zpk = None if sym else O.pack_zeros(c.zp)
        y1 = O.linear_ref(c.x_bits, O.pack_weights(c.q), c.s_bits, zpk, c.bias_bits,
                          3, 16, 384, 384, dt)
        s3 = np.repeat(c.s_bits, 3, axis=1)
        z3 = None if sym else O.pack_zeros(np.repeat(c.zp, 3, axis=1))
        y3 = O.linear_ref(c.x_bits, O.pack_weights(c.q), s3, z3, c.bias_bits, 3, 16, 384, 128, dt)
        assert np.array_equal(y1, y3)
        # and a changed scale moves every weight of its row, nowhere else
        s_b = c.s_bits.copy()
        s_b[5, 0] = O.f32_to_act_bits(np.float32(2.0) * O.act_bits_to_f64(s_b[5:6, 0], dt).astype(np.float32), dt)[0]
        W0 = O.dequant_f32(O.pack_weights(c.q), c.s_bits, zpk, 16, 384, 384, dt)
        W1 = O.dequant_f32(O.pack_weights(c.q), s_b, zpk, 16, 384, 384, dt)
        changed = np.argwhere(W0 != W1)
        assert set(changed[:, 0].tolist()) <= {5}
        assert np.array_equal(W1[5], 2.0 * W0[5])


def test_dequant_rejects_bad_group():
    with pytest.raises(ValueError):
        O.dequant_f32(np.zeros((8, 5), np.int32), np.zeros((8, 1), np.uint16), None, 8, 40, 32, O.F16)


# --------------------------------------------------------------------------
# expert-indexed product
# --------------------------------------------------------------------------

def _moe_stack(E, N, K, g, dt, sym, bias, seed):
    """E independent layers, and their stacks [E, ...] in the layer layouts."""
    cases = [make_case(1, N, K, g, dt, sym, bias, seed=(seed, e)) for e in range(E)]
    wq = np.stack([O.pack_weights(c.q) for c in cases])
    s = np.stack([c.s_bits for c in cases])
    z = None if sym else np.stack([O.pack_zeros(c.zp) for c in cases])
    b = np.stack([c.bias_bits for c in cases]) if bias else None
    return cases, wq, s, z, b


def test_moe_single_expert_is_the_linear_layer():
    cases, wq, s, z, b = _moe_stack(1, 16, 256, 64, O.BF16, False, True, "moe1")
    x = make_case(3, 16, 256, 64, O.BF16, False, False, seed="moe1x").x_bits
    ids = np.zeros((3, 2), dtype=np.int32)
    y = O.moe_linear_ref(x, wq, s, z, b, ids, None, 3, 2, 1, 16, 256, 64, O.BF16)
    ref = O.linear_ref(x, wq[0], s[0], z[0], b[0], 3, 16, 256, 64, O.BF16)
    assert np.array_equal(y[0::2], ref) and np.array_equal(y[1::2], ref)


def test_moe_slot_uses_its_own_expert_slice():
    E, N, K = 4, 16, 128
    cases, wq, s, z, b = _moe_stack(E, N, K, 32, O.F16, False, True, "moe2")
    x = make_case(2, N, K, 32, O.F16, False, False, seed="moe2x").x_bits
    ids = np.array([[3, 0], [1, 3]], dtype=np.int32)
    y = O.moe_linear_ref(x, wq, s, z, b, ids, None, 2, 2, E, N, K, 32, O.F16)
    for m in range(2):
        for j in range(2):
            e = ids[m, j]
            c = cases[e]
            ref = O.linear_ref(x[m:m + 1], O.pack_weights(c.q), c.s_bits, O.pack_zeros(c.zp),
                               c.bias_bits, 1, N, K, 32, O.F16)[0]
            assert np.array_equal(y[m * 2 + j], ref)
    # relabelling the experts (stacks permuted, ids mapped) changes nothing
    perm = np.array([2, 0, 3, 1])
    inv = np.argsort(perm)
    y2 = O.moe_linear_ref(x, wq[perm], s[perm], z[perm], b[perm], inv[ids], None,
                          2, 2, E, N, K, 32, O.F16)
    assert np.array_equal(y2, y)


def test_moe_weights_ids_and_slot_rows():
    E, N, K = 3, 8, 64
    cases, wq, s, z, b = _moe_stack(E, N, K, 32, O.BF16, True, False, "moe3")
    x = make_case(2, N, K, 32, O.BF16, True, False, seed="moe3x").x_bits
    ids = np.array([[0, 2], [1, 7]], dtype=np.int32)   # 7 is not an expert
    y = O.moe_linear_ref(x, wq, s, None, None, ids, None, 2, 2, E, N, K, 32, O.BF16)
    assert np.all(y[3] == 0.0) and np.any(y[2] != 0.0)
    w = np.array([[2.0, 0.0], [0.25, 1.0]], dtype=np.float32)
    yw = O.moe_linear_ref(x, wq, s, None, None, ids, w, 2, 2, E, N, K, 32, O.BF16)
    assert np.array_equal(yw[0], 2.0 * y[0]) and np.all(yw[1] == 0.0)
    assert np.array_equal(yw[2], 0.25 * y[2])
    # one x row per slot, equal to its token's row, is the shared-x product
    xs = np.repeat(np.asarray(x).reshape(2, K), 2, axis=0)
    ys = O.moe_linear_ref(xs, wq, s, None, None, ids, None, 2, 2, E, N, K, 32, O.BF16,
                          x_per_slot=True)
    assert np.array_equal(ys, y)


def test_complete_tiles_are_self_contained():
    # the rows of a complete 16-row tile (K a multiple of 128) hold exactly
    # that tile's codes: slicing the packed tensor at tile boundaries equals
    # packing the slice, and a tile's words unpack on their own
    rng = np.random.default_rng(5)
    N, K = 64, 512
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    wq = O.pack_weights(q)
    for t in range(N // 16):
        rows = slice(16 * t, 16 * t + 16)
        assert np.array_equal(wq[rows], O.pack_weights(q[rows]))
        assert np.array_equal(O.unpack_weights(wq[rows]), q[rows])
