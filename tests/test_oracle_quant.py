"""Pins for oracle.quant: scale invariants, error bounds, constructed exact ties,
saturation, zero rows/blocks, nibble order, the global-scale rule and the
SVDQuant smoothing division."""
from fractions import Fraction

import numpy as np

from oracle.formats import e2m1_decode, e4m3_decode, e4m3_encode, bf16_bits_to_f32
from oracle.quant import (amax_bf16, calibrate_input_scale, global_scale, pack_e2m1,
                          quant_fp8_row, quant_nvfp4, smooth_bf16, unpack_e2m1)
from synthetic import bf16_round, make, calibration_batches

F32 = np.float32


def rand_bf16(shape, seed, scale=1.0):
    return bf16_round(np.random.default_rng(seed).standard_normal(shape).astype(F32) * F32(scale))


# ---------------------------------------------------------------- fp8r

def test_fp8_row_max_code_is_448():
    x = make("fp8r_tiny")["x"]
    codes, s = quant_fp8_row(x)
    dec = np.abs(e4m3_decode(codes))
    assert np.all(s > 0)
    # the row maximum maps to 448 exactly (its neighbours are 416 and NaN)
    assert np.all(dec.max(axis=1) == 448.0)


def test_fp8_row_error_bound():
    x = rand_bf16((64, 512), 1, 3.0)
    codes, s = quant_fp8_row(x)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    q = xf / s[:, None].astype(np.float64)
    # half an E4M3 ulp at |q| (subnormal step 2^-9 below 2^-6), plus one fp32 rounding of q
    e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
    half_ulp = np.ldexp(0.5, (e - 3).astype(int))
    err = np.abs(q - e4m3_decode(codes))
    assert np.all(err <= half_ulp * (1 + 2.0 ** -20) + np.abs(q) * 2.0 ** -23)


def test_fp8_row_scale_rule():
    x = rand_bf16((16, 64), 2)
    _, s = quant_fp8_row(x)
    amax = np.abs(bf16_bits_to_f32(x)).max(axis=1)
    assert s.dtype == np.float32
    assert np.array_equal(s, (amax / F32(448)).astype(F32))


def test_fp8_row_zero_row_signed_zeros():
    x = np.zeros((2, 32), np.uint16)
    x[1, ::2] = 0x8000  # -0.0
    codes, s = quant_fp8_row(x)
    assert np.all(s == 0)
    assert np.all(codes[0] == 0) and np.all(codes[1, ::2] == 0x80) and np.all(codes[1, 1::2] == 0)


def test_fp8_row_exact_ties():
    # amax = 448 * 2^j gives s = 2^j, so x = midpoint * 2^j is an exact tie for the encoder
    pos = e4m3_decode(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2)
    rows = []
    for j in (-3, 0, 2):
        vals = np.ldexp(mids, j)
        vals = vals[(np.abs(vals) < 448 * 2.0 ** j)]
        row = np.concatenate([[448 * 2.0 ** j], vals, -vals]).astype(F32)
        b = bf16_round(row)
        keep = bf16_bits_to_f32(b) == row  # only exactly representable ties
        rows.append((j, b[keep]))
    for j, b in rows:
        codes, s = quant_fp8_row(b[None, :])
        assert s[0] == F32(2.0 ** j)
        c = codes[0, 1:].astype(int)
        assert np.all((c & 1) == 0), "ties must land on even codes"


def test_fp8_row_divides_rather_than_multiplies_by_reciprocal():
    # reading: codes come from x / s, correctly rounded; x * (1/s) differs on some ties
    x = make("fp8r_tiny")["x"]
    codes, s = quant_fp8_row(x)
    xf = bf16_bits_to_f32(x)
    by_div = e4m3_encode((xf / s[:, None]).astype(F32))
    assert np.array_equal(codes, by_div)
    big = rand_bf16((512, 3072), 11)
    c2, s2 = quant_fp8_row(big)
    xf2 = bf16_bits_to_f32(big)
    by_rcp = e4m3_encode((xf2 * (F32(1) / s2)[:, None]).astype(F32))
    assert np.count_nonzero(by_rcp != c2) > 0  # the two readings really differ


# ---------------------------------------------------------------- nvfp4

def test_global_scale_rule_and_calibration():
    assert global_scale(F32(2688)) == F32(1.0)
    assert global_scale(F32(5.25)) == F32(5.25) / F32(2688)
    batches = list(calibration_batches("svdq_w4a4", M=8, K=64))
    assert len(batches) == 8
    amaxes = [amax_bf16(b) for b in batches]
    assert calibrate_input_scale(batches) == F32(max(amaxes)) / F32(2688)


def test_nvfp4_block_max_maps_to_six():
    x = rand_bf16((32, 256), 4)
    g = global_scale(amax_bf16(x))
    packed, sf = quant_nvfp4(x, g)
    codes = unpack_e2m1(packed).reshape(32, 16, 16)
    xb = np.abs(bf16_bits_to_f32(x)).reshape(32, 16, 16)
    u = (xb.max(axis=2) / (F32(6) * g)).astype(F32)
    normal = (u >= 2.0 ** -6) & (u <= 448)
    top = np.abs(e2m1_decode(codes)).max(axis=2)
    assert normal.sum() > 400
    assert np.all(top[normal] == 6.0)


def test_nvfp4_exact_ties():
    # g = 0.25, block max 6 -> sf = E4M3(6 / 1.5) = 4.0, d = 1.0: midpoints are exact ties
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = np.array([6.0] + ties + [-t for t in ties] + [0.0], dtype=F32)
    packed, sf = quant_nvfp4(bf16_round(row)[None, :], F32(0.25))
    assert e4m3_decode(sf[0, 0]) == 4.0
    vals = e2m1_decode(unpack_e2m1(packed)[0])
    assert np.array_equal(vals[1:8], expect)
    assert np.array_equal(vals[8:15], [-e for e in expect])


def test_nvfp4_saturation_and_zero_block():
    # block 0: bmax / (6 g) far above 448 -> sf = 448 and codes clamp at +-6
    # block 1: all zeros (with -0) -> sf = 0 and signed-zero codes
    row = np.zeros(32, F32)
    row[:16] = np.linspace(-5000, 5000, 16, dtype=F32)
    x = bf16_round(row)[None, :]
    x[0, 17] = 0x8000
    packed, sf = quant_nvfp4(x, F32(0.01))
    assert sf[0, 0] == 0x7E and sf[0, 1] == 0
    c = unpack_e2m1(packed)[0]
    assert np.abs(e2m1_decode(c[:16])).max() == 6.0 and e2m1_decode(c[0]) == -6.0
    assert np.all((c[16:] & 7) == 0) and c[17] == 0x8 and c[16] == 0x0


def test_nvfp4_error_bound_unsaturated():
    x = rand_bf16((16, 512), 5)
    g = global_scale(amax_bf16(x))
    packed, sf = quant_nvfp4(x, g)
    d = (e4m3_decode(sf).astype(F32) * g).astype(F32).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64).reshape(16, 32, 16)
    q = xf / d[:, :, None]
    v = e2m1_decode(unpack_e2m1(packed)).reshape(16, 32, 16)
    ok = np.abs(q) <= 6.0
    e = np.floor(np.log2(np.maximum(np.abs(q), 1.0)))
    half_ulp = np.ldexp(0.25, e.astype(int))
    assert np.all((np.abs(q - v) <= half_ulp * (1 + 2.0 ** -20) + np.abs(q) * 2.0 ** -23)[ok])


def test_nibble_order_low_is_even():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    p = pack_e2m1(codes)
    assert p.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(unpack_e2m1(p), codes)


def test_nvfp4_weight_global_scale_saturates_nothing():
    w = make("nvfp4_dit", M=8, K=256, N=64)["w"]
    g = global_scale(amax_bf16(w))
    _, sf = quant_nvfp4(w, g)
    assert int(sf.max()) <= 0x7E
    # the tensor maximum sits in a block whose scale is 448 (code 0x7E) or just below
    assert e4m3_decode(sf).max() >= 416.0


# ---------------------------------------------------------------- smoothing

def test_smooth_unit_factor_is_identity():
    x = rand_bf16((8, 64), 11, 3.0)
    x[0, :4] = [0x0000, 0x8000, 0x0001, 0x8001]  # signed zeros and bf16 subnormals
    assert np.array_equal(smooth_bf16(x, np.ones(64, F32)), x)


def test_smooth_power_of_two_shifts_the_exponent():
    # x / 2^j is exact; on bf16 bit patterns it subtracts j from the exponent field
    rng = np.random.default_rng(12)
    x = rand_bf16((16, 48), 12, 1.0)
    x[x & 0x7F80 == 0] = 0x3F80  # keep every value normal and away from the edges
    j = rng.integers(-8, 9, size=48)
    lam = np.ldexp(np.ones(48), j).astype(F32)
    expect = (x.astype(np.int64) - (j[None, :] << 7)).astype(np.uint16)
    assert np.array_equal(smooth_bf16(x, lam), expect)


def _round_rne(q, p):
    """Nearest value with p significant bits to the nonzero rational q, ties to even
    (normal range only)."""
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    unit = Fraction(2) ** (e - p + 1)
    n = a // unit
    rem = a - n * unit
    if rem > unit / 2 or (rem == unit / 2 and n % 2 == 1):
        n += 1
    v = n * unit
    return v if q > 0 else -v


def test_smooth_is_fp32_division_then_bf16_rounding():
    # brute force from exact rationals: round x / lam to 24 significant bits, then to 8
    rng = np.random.default_rng(13)
    x = rand_bf16((1, 400), 13, 4.0)[0]
    x[x & 0x7F80 == 0] = 0xC0A0
    lam = np.exp(rng.uniform(-6, 6, size=400)).astype(F32)
    lam[:40] = np.nextafter(np.ldexp(F32(1), rng.integers(-5, 6, size=40)).astype(F32), F32(0))  # 1.11..1 x 2^e
    lam[40:80] = (F32(1) + F32(2.0 ** -23) * rng.integers(1, 64, size=40)).astype(F32)
    # factors whose quotient lies just off a bf16 midpoint: there the two roundings
    # differ from one rounding of the exact quotient
    xs, ls = [], []
    for _ in range(64):
        xb = int(rng.integers(0x3F80, 0x4000))
        xf = float(np.array([xb << 16], np.uint32).view(F32)[0])
        m = Fraction(1) + Fraction(2 * int(rng.integers(0, 128)) + 1, 256)
        c = F32(float(Fraction(xf) / m))
        xs += [xb] * 3
        ls += [c, np.nextafter(c, F32(0)), np.nextafter(c, F32(10))]
    x = np.concatenate([x, np.array(xs, np.uint16)])
    lam = np.concatenate([lam, np.array(ls, F32)])
    got = smooth_bf16(x[None, :], lam)[0]
    xv = bf16_bits_to_f32(x)
    double = 0
    for i in range(x.size):
        q = Fraction(float(xv[i])) / Fraction(float(lam[i]))
        q8 = _round_rne(_round_rne(q, 24), 8)
        double += q8 != _round_rne(q, 8)
        assert Fraction(float(bf16_bits_to_f32(got[i:i + 1])[0])) == q8, (i, xv[i], lam[i])
    assert double >= 4


def test_smooth_divides_and_the_weight_multiplies():
    # SVDQuant moves a channel's range from x into W: (x / lam) (W lam)^T = x W^T.
    # With power-of-two factors every step is exact, so the identity holds exactly;
    # a multiplication by lam in place of the division fails it.
    rng = np.random.default_rng(14)
    xi = rng.integers(-8, 9, size=(6, 32)).astype(F32)
    wi = rng.integers(-8, 9, size=(5, 32)).astype(np.float64)
    lam = np.ldexp(np.ones(32), rng.integers(-3, 4, size=32)).astype(F32)
    x_bits = (xi.view(np.uint32) >> 16).astype(np.uint16)
    xh = bf16_bits_to_f32(smooth_bf16(x_bits, lam)).astype(np.float64)
    assert np.array_equal(xh @ (wi * lam.astype(np.float64)[None, :]).T, xi.astype(np.float64) @ wi.T)
    assert not np.array_equal(xh, xi.astype(np.float64))


def test_smooth_keeps_signs():
    x = np.array([[0x8000, 0x0000, 0xBF80, 0x3F80]], np.uint16)
    got = smooth_bf16(x, np.array([3.0, 3.0, 7.0, 7.0], F32))
    assert got[0, 0] == 0x8000 and got[0, 1] == 0x0000
    assert got[0, 2] & 0x8000 and not got[0, 3] & 0x8000
    assert got[0, 2] == got[0, 3] | 0x8000
