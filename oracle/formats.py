"""Element formats: E4M3, E2M1 and bf16 (oracle; test infrastructure only).

The BFL guide's intro bullets name the formats but do not define them.  The
readings taken here:

* E4M3 is the OCP 8-bit floating point "E4M3" encoding (OCP OFP8 spec, rev 1.0):
  1 sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals, no infinity,
  NaN only at S.1111.111, largest finite magnitude 448.
* E2M1 is the OCP Microscaling "FP4 E2M1" element type (OCP MX spec v1.0):
  1 sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* Encoding rounds to nearest, ties to the even code (IEEE roundTiesToEven),
  saturates at the largest finite magnitude (never produces NaN), and keeps the
  sign of zero and of values that underflow to zero.
* Inputs are finite; NaN and infinity are outside the contract.
"""
import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _split_sign(v):
    v = np.asarray(v, dtype=np.float32)
    return np.signbit(v), np.abs(v).astype(np.float64)


def _encode_minifloat(a, mbits, bias, min_normal_exp, sat_code, sat_value):
    """Round non-negative float64 magnitudes ``a`` (exact copies of float32
    values) to a minifloat with ``mbits`` mantissa bits; returns magnitude codes.

    Normal range: a = 2**e * (1 + m / 2**mbits), code = (e + bias) << mbits | m.
    Subnormal range (a < 2**min_normal_exp): multiples of 2**(min_normal_exp - mbits);
    code = rint(a / that step), where the value 2**mbits lands on the first normal.
    All scalings are by powers of two, so every step before ``rint`` is exact.
    """
    code = np.zeros(a.shape, dtype=np.int64)
    sat = a >= sat_value
    sub = (~sat) & (a < 2.0 ** min_normal_exp)
    nrm = ~(sat | sub)
    step_exp = min_normal_exp - mbits
    code[sub] = np.rint(np.ldexp(a[sub], -step_exp)).astype(np.int64)
    an = a[nrm]
    _, ex = np.frexp(an)            # an = f * 2**ex with f in [0.5, 1)
    e = ex.astype(np.int64) - 1     # floor(log2(an))
    frac = np.ldexp(an, -e) - 1.0   # in [0, 1), exact
    m = np.rint(np.ldexp(frac, mbits)).astype(np.int64)
    carry = m == (1 << mbits)
    e = e + carry
    m = np.where(carry, 0, m)
    code[nrm] = ((e + bias) << mbits) | m
    code[sat] = sat_code
    return code


def e4m3_encode(v):
    """float32 values -> E4M3 codes (uint8): RNE, saturating at 448, signed zero."""
    sign, a = _split_sign(v)
    mag = _encode_minifloat(a, mbits=3, bias=7, min_normal_exp=-6, sat_code=0x7E, sat_value=E4M3_MAX)
    return (mag | (sign.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(c):
    """E4M3 codes -> float64 values (exact).  0x7F / 0xFF decode to NaN."""
    c = np.asarray(c, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e2m1_encode(v):
    """float32 values -> E2M1 codes (uint8 in 0..15; bit 3 is the sign):
    RNE to {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6."""
    sign, a = _split_sign(v)
    mag = _encode_minifloat(a, mbits=1, bias=1, min_normal_exp=0, sat_code=7, sat_value=E2M1_MAX)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(c):
    """E2M1 codes (0..15) -> float64 values (exact)."""
    c = np.asarray(c, dtype=np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    val = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return s * val


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs).

    Written as the rounding rule on the 16 discarded bits: keep the upper half,
    add one when the discarded half is above 0x8000, or equal to it with the
    kept half odd.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    return (hi + up).astype(np.uint16)
