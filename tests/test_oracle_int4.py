"""Pins for oracle.int4 (group-wise symmetric INT4): the group max maps to +-7,
grid values round-trip, the rounding bound, constructed exact ties, two's
complement nibbles and their order, zero groups, and a brute-force dot product."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.formats import bf16_bits_to_f32
from oracle.int4 import dequant_int4, qlinear_int4_ref, quant_int4, unpack_int4
from synthetic import bf16_round, make

F32 = np.float32


def bits(v):
    return bf16_round(np.asarray(v, dtype=F32))


def test_group_max_maps_to_seven():
    x = make("svdq_w4a4", M=16, K=512)["x"]
    packed, s = quant_int4(x)
    q = unpack_int4(packed).reshape(16, 8, 64)
    xv = bf16_bits_to_f32(x).reshape(16, 8, 64)
    assert np.all(s > 0)
    assert np.all(np.abs(q).max(axis=2) == 7)
    at = np.abs(xv).argmax(axis=2)
    qa = np.take_along_axis(q, at[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(qa) == 7)


def test_grid_values_round_trip():
    rng = np.random.default_rng(1)
    R, G = 6, 5
    e = rng.integers(-20, 10, size=(R, G))
    q = rng.integers(-7, 8, size=(R, G, 64))
    q[:, :, 3] = np.where(rng.random((R, G)) < 0.5, 7, -7)
    x = (q * np.ldexp(1.0, e)[:, :, None]).reshape(R, G * 64)
    packed, s = quant_int4(bits(x))
    assert np.array_equal(s, np.ldexp(1.0, e).astype(F32))
    assert np.array_equal(unpack_int4(packed), q.reshape(R, -1).astype(np.int8))
    assert np.array_equal(dequant_int4(packed, s), x)


def test_rounding_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32, 256)) * np.exp(rng.uniform(-30, 30, size=(32, 1)))
    b = bits(x)
    xv = bf16_bits_to_f32(b).astype(np.float64)
    packed, s = quant_int4(b)
    d = dequant_int4(packed, s)
    sg = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(xv - d) <= sg * (0.5 + 2.0 ** -20))


def test_exact_ties_round_to_even():
    # group max 7 * 2^e makes s = 2^e; values (k + 1/2) 2^e are exact ties
    e = -3
    x = np.zeros((1, 64))
    x[0, 0] = 7 * 2.0 ** e
    halves = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5])
    x[0, 1:8] = halves * 2.0 ** e
    x[0, 8:15] = -halves * 2.0 ** e
    packed, s = quant_int4(bits(x))
    q = unpack_int4(packed)[0]
    assert s[0, 0] == F32(2.0 ** e)
    assert list(q[1:8]) == [0, 2, 2, 4, 4, 6, 6]
    assert list(q[8:15]) == [0, -2, -2, -4, -4, -6, -6]


def test_twos_complement_nibbles_low_is_even():
    x = np.zeros((1, 64))
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 7.0, -1.0, -7.0, 3.0
    packed, s = quant_int4(bits(x))
    assert s[0, 0] == 1.0
    assert packed[0, 0] == (0x7 | (0xF << 4))       # 7 low, -1 high
    assert packed[0, 1] == (0x9 | (0x3 << 4))       # -7 low, 3 high
    assert list(unpack_int4(np.array([[0x08]], np.uint8))[0]) == [-8, 0]


def test_zero_group():
    x = np.zeros((2, 128))
    x[1, 64:] = 1.0
    x[0, 5] = -0.0
    packed, s = quant_int4(bits(x))
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(packed[0] == 0) and np.all(packed[1, :32] == 0)


@pytest.mark.parametrize("M,K,N", [(3, 64, 4), (2, 192, 3)])
def test_gemm_brute_force(M, K, N):
    # y[m, n] = sum_g s_x[m, g] s_w[n, g] sum_{k in g} q_x q_w, summed exactly
    rng = np.random.default_rng(M * K + N)
    xp, xs = quant_int4(bits(rng.standard_normal((M, K))))
    wp, ws = quant_int4(bits(rng.standard_normal((N, K)) * 0.02))
    y = qlinear_int4_ref(xp, xs, wp, ws)
    qx, qw = unpack_int4(xp), unpack_int4(wp)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(K // 64):
                dot = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(64 * g, 64 * g + 64))
                acc += Fraction(float(xs[m, g])) * Fraction(float(ws[n, g])) * dot
            assert abs(float(acc) - y[m, n]) <= 1e-12 * max(1.0, abs(float(acc)))


def _rne_fraction_to_f32(q):
    """Nearest float32 to the positive rational q (normal range), ties to even."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    unit = Fraction(2) ** (e - 23)
    n = q // unit
    rem = q - n * unit
    if rem > unit / 2 or (rem == unit / 2 and n % 2 == 1):
        n += 1
    return n * unit


def test_divides_rather_than_multiplies_by_reciprocal():
    # near a half-integer x/s and x * RN(1/s) can round to different codes: the
    # code is rint of the correctly rounded quotient, computed here from rationals
    rng = np.random.default_rng(9)
    cases = []
    while len(cases) < 6:
        ab = int(rng.integers(0x3F80, 0x4100))
        amax = np.array([ab << 16], np.uint32).view(F32)[0]
        s = F32(amax / F32(7))
        r = F32(F32(1) / s)
        k = int(rng.integers(0, 7))
        xb = int(np.array([(k + 0.5) * float(s)], F32).view(np.uint32)[0] >> 16)
        for d in (-1, 0, 1):
            x = np.array([(xb + d) << 16], np.uint32).view(F32)[0]
            if x <= amax and np.rint(F32(x * r)) != np.rint(F32(x / s)):
                cases.append((ab, xb + d))
    for ab, xb in cases:
        row = np.zeros((1, 64), np.uint16)
        row[0, 0], row[0, 1] = ab, xb
        packed, s = quant_int4(row)
        xv = Fraction(float(bf16_bits_to_f32(np.array([xb], np.uint16))[0]))
        quot = _rne_fraction_to_f32(xv / Fraction(float(s[0, 0])))
        fl = quot.numerator // quot.denominator
        frac = quot - fl
        code = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1) else 0)
        assert unpack_int4(packed)[0, 1] == code, (hex(ab), hex(xb))
