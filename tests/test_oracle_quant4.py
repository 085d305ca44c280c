"""Pins of the quantized-base oracle (4-bit codes, one scale per 64-element row
block) against what its definition fixes by hand: packed bytes of a worked
row, exact round trips of representable matrices, the half-scale error bound,
zero blocks, and the sign/nibble order of the packing."""
import numpy as np
import pytest

import oracle as O


def test_worked_row_packing():
    # one block: w = 0.25 * [7, -7, 3, -1, 0, 5, -8/8*7 ...]; scale = 7*0.25/7 = 0.25
    q = np.zeros(64, dtype=np.int64)
    q[:6] = [7, -7, 3, -1, 0, 5]
    W = (q * 0.25)[None, :]
    codes, scales = O.quantize_int4_rows(W)
    assert scales.shape == (1, 1) and scales[0, 0] == np.float32(0.25)
    # byte j = low nibble of element 2j | high nibble of element 2j+1 (two's complement)
    assert codes[0, 0] == 0x97          # 7 -> 0x7, -7 -> 0x9
    assert codes[0, 1] == 0xF3          # 3 -> 0x3, -1 -> 0xF
    assert codes[0, 2] == 0x50          # 0 -> 0x0, 5 -> 0x5
    assert np.all(codes[0, 3:] == 0)
    assert np.array_equal(O.dequantize_int4_rows(codes, scales), W)


def test_nibble_sign_decoding():
    codes = np.array([[0x8F, 0x70, 0x01]], dtype=np.uint8)
    assert O.int4_codes(codes).tolist() == [[-1, -8, 0, 7, 1, 0]]


def test_representable_matrices_round_trip_exactly():
    rng = np.random.default_rng(3)
    rows, cols = 5, 256
    q = rng.integers(-7, 8, size=(rows, cols))
    q[:, ::64] = 7                                    # every block reaches |q| = 7
    s = 2.0 ** rng.integers(-12, 2, size=(rows, cols // 64))
    W = q * np.repeat(s, 64, axis=1)
    codes, scales = O.quantize_int4_rows(W)
    assert np.array_equal(scales.astype(np.float64), s)
    assert np.array_equal(O.int4_codes(codes), q)
    assert np.array_equal(O.dequantize_int4_rows(codes, scales), W)


def test_error_within_half_a_step():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((7, 512)) * rng.lognormal(0, 2, (7, 1))
    codes, scales = O.quantize_int4_rows(W)
    step = np.repeat(scales.astype(np.float64), 64, axis=1)
    err = np.abs(O.dequantize_int4_rows(codes, scales) - W)
    assert np.all(err <= step / 2 + 1e-6 * np.abs(W))
    # the block maximum is always coded as +-7
    q = np.abs(O.int4_codes(codes)).reshape(7, 8, 64)
    assert np.all(q.max(axis=2) == 7)


def test_zero_blocks_and_width_check():
    W = np.zeros((2, 128))
    W[1, 64:] = -3.0
    codes, scales = O.quantize_int4_rows(W)
    assert scales[0].tolist() == [0.0, 0.0] and scales[1, 0] == 0.0
    assert np.all(O.int4_codes(codes)[1, 64:] == -7)
    deq = O.dequantize_int4_rows(codes, scales)
    assert np.all(deq[0] == 0.0) and np.all(deq[1, :64] == 0.0)          # zero blocks stay exactly zero
    assert np.allclose(deq[1, 64:], -3.0, rtol=0, atol=float(scales[1, 1]) / 2)
    with pytest.raises(ValueError):
        O.quantize_int4_rows(np.zeros((1, 100)))


# The code is an integer decided by floating point; the pages fix no precision,
# so the reading is IEEE fp32 (s = fp32(max|w| / 7), q = rint(fp32(w / s)), ties
# to even).  These elements pin that reading against exact rational arithmetic:
# with max|w| = 1 the scale is fp32(1/7) = 9586981 / 2^26, and the two weights
# below have fp32 quotients exactly 1.5 and 4.5 (codes 2 and 4 by ties to even)
# while their exact quotients, 1.49999995 and 4.50000016, round to 1 and 5.
from fractions import Fraction


def _round_fp32(x: Fraction) -> Fraction:
    """Nearest fp32 value of a rational (normal range), ties to even."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    return sgn * _rint_even(a / ulp) * ulp


def _rint_even(x: Fraction) -> int:
    f = x.numerator // x.denominator          # floor
    rem = x - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def test_code_decided_in_fp32_with_ties_to_even():
    w_tie_lo = np.float32(0.2142857164144516)
    w_tie_hi = np.float32(0.6428571939468384)
    rng = np.random.default_rng(5)
    row = (rng.standard_normal(64) * 0.3).astype(np.float32)
    row[0] = np.float32(1.0)                 # block maximum
    row[1], row[2] = w_tie_lo, w_tie_hi
    row[3], row[4] = -w_tie_lo, -w_tie_hi
    codes, scales = O.quantize_int4_rows(row[None, :])
    s = _round_fp32(Fraction(1) / 7)
    assert Fraction(float(scales[0, 0])) == s
    expect = [max(-7, min(7, _rint_even(_round_fp32(Fraction(float(w)) / s)))) for w in row]
    assert O.int4_codes(codes)[0].tolist() == expect
    assert expect[1:5] == [2, 4, -2, -4]
    # the exact quotient would decide differently: the pin separates the readings
    assert [_rint_even(Fraction(float(w)) / s) for w in row[1:3]] == [1, 5]
